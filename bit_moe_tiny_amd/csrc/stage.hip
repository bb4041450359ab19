// Activation staging: rows -> fp16 images for the matrix-core kernels.
//
// Every verifier row is tiny (hidden <= 16384 values) next to the weights it
// meets, so it is prepared once per call: scaled by a power of two so its
// largest magnitude lies in [2^10, 2^11) (keeps every fp16 product and the
// 16-element sums far from overflow), split into an fp16 high part and an
// fp16 remainder (together ~22 significant bits; an fp32 row survives to well
// inside the 2e-3 output bound, a bf16 row is exact in the high part alone),
// and laid out in the order the consuming kernel unpacks weights.
#include "sv_internal.h"
#include "sv_stage.h"

namespace sv {

__global__ __launch_bounds__(256) void k_stage(const void* src, int dtype, int K, int layout,
                                               const int* n_rows_dev, XImg img) {
  extern __shared__ float xs[];
  __shared__ float red[4];
  __shared__ int flag[4];
  const int row = blockIdx.x;
  if (n_rows_dev && row >= *n_rows_dev) return;
  stage_row(src, dtype, (size_t)row * K, row, K, layout, img, xs, red, flag);
}

hipError_t launch_stage(const void* src, int dtype, int rows, int K, int layout,
                        const int* n_rows_dev, XImg img, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_stage, dim3(rows), dim3(256), (size_t)K * sizeof(float), s, src, dtype,
                     K, layout, n_rows_dev, img);
  return hipGetLastError();
}

}  // namespace sv

// Activation staging: rows -> fp16 images for the matrix-core kernels.
//
// Every verifier row is tiny (hidden <= 16384 values) next to the weights it
// meets, so it is prepared once per call: each 256-element block is scaled by a
// power of two (block max in [2^10, 2^11)), split into an fp16 high part and an
// fp16 remainder (together ~22 significant bits; a bf16 row is exact in the
// high part alone), and laid out in the order the consuming kernel unpacks
// weights.  One half-wave per (row, block): a single parallel pass.
#include "sv_internal.h"
#include "sv_stage.h"

namespace sv {

template <int DT>
__global__ __launch_bounds__(256) void k_stage(const void* src, int rows, int layout,
                                               const int* n_rows_dev, XImg img) {
  const int n_rows = n_rows_dev ? *n_rows_dev : rows;
  stage_gid<DT>(src, n_rows, layout, img, blockIdx.x * 8 + (threadIdx.x >> 5), threadIdx.x & 31);
}

hipError_t launch_stage(const void* src, int dtype, int rows, int K, int layout,
                        const int* n_rows_dev, XImg img, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int groups = rows * ((K + 255) / 256);
  if (dtype == SV_BF16)
    hipLaunchKernelGGL(k_stage<SV_BF16>, dim3((groups + 7) / 8), dim3(256), 0, s, src, rows,
                       layout, n_rows_dev, img);
  else
    hipLaunchKernelGGL(k_stage<SV_F32>, dim3((groups + 7) / 8), dim3(256), 0, s, src, rows, layout,
                       n_rows_dev, img);
  return hipGetLastError();
}

}  // namespace sv

// Activation staging: rows -> fp16 images for the matrix-core kernels.
//
// Every verifier row is tiny (hidden <= 16384 values) next to the weights it
// meets, so it is prepared once per call: the row is scaled by a power of two
// (row max in [2^10, 2^11)), split into an fp16 high part and an fp16
// remainder (together ~22 significant bits; a bf16 row is exact in the high
// part alone), and laid out in the order the consuming kernel unpacks
// weights.  One thread block per row.
#include "sv_internal.h"
#include "sv_stage.h"

namespace sv {

constexpr int STAGE_THREADS = 1024;

template <int DT>
__global__ __launch_bounds__(STAGE_THREADS) void k_stage(const void* src, int rows, int layout,
                                               const int* n_rows_dev, XImg img) {
  __shared__ int sh[2 * STAGE_THREADS / 64];
  const int n_rows = n_rows_dev ? *n_rows_dev : rows;
  if ((int)blockIdx.x >= n_rows) return;
  stage_row<DT, STAGE_THREADS>(src, blockIdx.x, layout, img, sh);
}

hipError_t launch_stage(const void* src, int dtype, int rows, int K, int layout,
                        const int* n_rows_dev, XImg img, hipStream_t s) {
  (void)K;
  if (rows <= 0) return hipSuccess;
  if (dtype == SV_BF16)
    hipLaunchKernelGGL(k_stage<SV_BF16>, dim3(rows), dim3(STAGE_THREADS), 0, s, src, rows, layout,
                       n_rows_dev, img);
  else
    hipLaunchKernelGGL(k_stage<SV_F32>, dim3(rows), dim3(STAGE_THREADS), 0, s, src, rows, layout,
                       n_rows_dev, img);
  return hipGetLastError();
}

}  // namespace sv

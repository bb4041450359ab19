// Test exports: dequantised weights as fp32.
//
// Two-bit: both products d*(sc*q) and dmin*m are exact in fp32 (11-bit fp16
// significand times a <= 6-bit integer), so the one fused multiply-add below
// rounds the exact weight d*sc*q - dmin*m once, to nearest-even -- the
// canonical dequantised value (an exact zero is +0).  Eight-bit: d*q is exact.
#include "sv_internal.h"

namespace sv {

__device__ inline float h16(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

__global__ __launch_bounds__(256) void k_q2_dequant(Q2View W, int k_in, float* out) {
  const size_t total = (size_t)W.n_out * k_in;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (size_t)gridDim.x * 256) {
    const size_t n = i / k_in, k = i - n * k_in;
    const size_t b = n * W.nb + k / 256;
    const int e = (int)(k & 255);
    const int q = (W.qs[b * 64 + e / 4] >> (2 * (e & 3))) & 3;
    const int nib = W.sc[b * 16 + e / 16];
    const float sc = (float)(nib & 15), m = (float)(nib >> 4);
    // "+ 0.0f" turns an exact zero into +0 whatever the signs of d and dmin
    out[i] = fmaf(h16(W.d[b]), sc * (float)q, -(h16(W.dm[b]) * m)) + 0.0f;
  }
}

__global__ __launch_bounds__(256) void k_q8_dequant(Q8View W, int k_in, float* out) {
  const size_t total = (size_t)W.n_out * k_in;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (size_t)gridDim.x * 256) {
    const size_t n = i / k_in, k = i - n * k_in;
    const size_t b = n * W.nb + k / 32;
    out[i] = h16(W.d[b]) * (float)W.qs[b * 32 + (k & 31)];
  }
}

static dim3 grid_for(size_t total) {
  size_t g = (total + 255) / 256;
  if (g > 65536) g = 65536;
  if (g == 0) g = 1;
  return dim3((unsigned)g);
}

hipError_t launch_q2_dequant(const void* w, int n_out, int k_in, float* out, hipStream_t s) {
  hipLaunchKernelGGL(k_q2_dequant, grid_for((size_t)n_out * k_in), dim3(256), 0, s,
                     q2_view(w, n_out, k_in), k_in, out);
  return hipGetLastError();
}

hipError_t launch_q8_dequant(const void* w, int n_out, int k_in, float* out, hipStream_t s) {
  hipLaunchKernelGGL(k_q8_dequant, grid_for((size_t)n_out * k_in), dim3(256), 0, s,
                     q8_view(w, n_out, k_in), k_in, out);
  return hipGetLastError();
}

}  // namespace sv

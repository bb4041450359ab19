// Eight-bit vocabulary head: logits[R, vocab] = W[vocab x hidden] h, each
// weight tile read once from HBM and reused for all R rows ("Q8 tiny-batch
// reuse", GB10/GX10 DSpark thread, post 1).
//
// v_mfma_f32_16x16x32_f16 with A = staged rows (lane: column c = lane&15,
// k-group g = lane>>4, 8 consecutive k), B = weights (lane: vocab row
// n = lane&15, bytes 8g..8g+7 of one 32-code block).  One instruction covers
// exactly one block of 16 vocab rows, so its result is scaled by each row's
// block scale in fp32 right away.  int8 codes become exact fp16 integers
// without conversion instructions: flipping the sign bit gives q+128 as a
// byte, which placed under the exponent of 1024.0 reads as 1152+q; one packed
// subtract leaves q.
#include "sv_internal.h"

namespace sv {

__device__ inline float f16b_to_f32(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

__device__ inline h2_t bytes01_to_h2(uint32_t u) {
  return __builtin_bit_cast(h2_t, (u & 0xFFu) | ((u & 0xFF00u) << 8) | 0x64006400u);
}
__device__ inline h2_t bytes23_to_h2(uint32_t u) {
  return __builtin_bit_cast(h2_t, ((u >> 16) & 0xFFu) | ((u >> 8) & 0xFF0000u) | 0x64006400u);
}

__device__ inline h8_t q8_bop(uint2 q) {
  const uint32_t a = q.x ^ 0x80808080u, b = q.y ^ 0x80808080u;
  const h2_t off = {(_Float16)1152.f, (_Float16)1152.f};
  const h2_t p0 = bytes01_to_h2(a) - off, p1 = bytes23_to_h2(a) - off;
  const h2_t p2 = bytes01_to_h2(b) - off, p3 = bytes23_to_h2(b) - off;
  h8_t r = {p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
  return r;
}

template <bool USE_LO, int T>
__global__ __launch_bounds__(256) void k_q8_lmhead(Q8View W, int R, XImg img, float* logits) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int tile0 = (blockIdx.x * 4 + wv) * T;
  const int vocab = W.n_out, K = W.nb * 32;
  if (tile0 * 16 >= vocab) return;
  const int nl = lane & 15, g = lane >> 4, cg = blockIdx.z;
  const int c = cg * 16 + nl;
  const _Float16* xh = c < R ? img.hi + (size_t)c * K : nullptr;
  const _Float16* xl = c < R ? img.lo + (size_t)c * K : nullptr;
  int nrow[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int n = (tile0 + t) * 16 + nl;
    nrow[t] = n < vocab ? n : vocab - 1;   // ragged tail: valid row, result dropped
  }
  const f4_t zero = {0.f, 0.f, 0.f, 0.f};
  const h8_t z8 = {0, 0, 0, 0, 0, 0, 0, 0};
  f4_t acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = zero;
  for (int kb = 0; kb < W.nb; ++kb) {
    const h8_t a = xh ? *(const h8_t*)(xh + kb * 32 + 8 * g) : z8;
    h8_t al = z8;
    if (USE_LO) al = xl ? *(const h8_t*)(xl + kb * 32 + 8 * g) : z8;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const size_t b = (size_t)nrow[t] * W.nb + kb;
      const uint2 q = *(const uint2*)(W.qs + b * 32 + 8 * g);
      const float d = f16b_to_f32(W.d[b]);
      const h8_t bw = q8_bop(q);
      f4_t dt = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bw, zero, 0, 0, 0);
      if (USE_LO) dt = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bw, dt, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[t][e] = fmaf(d, dt[e], acc[t][e]);
    }
  }
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int n = (tile0 + t) * 16 + nl;
    if (n >= vocab) continue;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int cc = cg * 16 + 4 * g + e;
      if (cc < R) logits[(size_t)cc * vocab + n] = acc[t][e] * img.rscale[cc];
    }
  }
}

constexpr int LM_T = 2;

hipError_t launch_q8_lmhead(const void* w, int vocab, int hidden, int R, bool use_lo, XImg img,
                            float* logits, hipStream_t s) {
  const Q8View W = q8_view(w, vocab, hidden);
  const int tiles = (vocab + 15) / 16;
  const int waves = (tiles + LM_T - 1) / LM_T;
  const dim3 grid((waves + 3) / 4, 1, (R + 15) / 16);
  if (use_lo)
    hipLaunchKernelGGL((k_q8_lmhead<true, LM_T>), grid, dim3(256), 0, s, W, R, img, logits);
  else
    hipLaunchKernelGGL((k_q8_lmhead<false, LM_T>), grid, dim3(256), 0, s, W, R, img, logits);
  return hipGetLastError();
}

}  // namespace sv

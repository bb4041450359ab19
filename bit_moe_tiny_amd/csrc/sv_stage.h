// Device routines that stage activation rows into an XImg (layout and scaling
// described in sv_internal.h).  One thread block per row: a first pass finds
// the row's largest magnitude (its power-of-two scale), a second pass converts
// the row block by block, 32 lanes -- half a wave -- per 256-element block,
// each lane converting 8 elements.
#pragma once

#include "sv_internal.h"

namespace sv {

template <int DT>
__device__ __forceinline__ void load4_act(const void* src, size_t idx, float* v) {
  if (DT == SV_BF16) {
    const uint2 b = *(const uint2*)((const uint16_t*)src + idx);
    v[0] = __uint_as_float(b.x << 16);
    v[1] = __uint_as_float(b.x & 0xFFFF0000u);
    v[2] = __uint_as_float(b.y << 16);
    v[3] = __uint_as_float(b.y & 0xFFFF0000u);
  } else {
    const float4 f = *(const float4*)((const float*)src + idx);
    v[0] = f.x;
    v[1] = f.y;
    v[2] = f.z;
    v[3] = f.w;
  }
}

__device__ __forceinline__ void split16(float v, _Float16& hi, _Float16& lo) {
  hi = (_Float16)v;
  lo = (_Float16)(v - (float)hi);
}

// Power-of-two exponent that puts a row's largest magnitude mx in
// [2^10, 2^11); 0 for an all-zero or non-finite row (then nothing is scaled
// and the non-finite values propagate as they are).
__device__ __forceinline__ int row_exponent(float mx, int bad) {
  int esc = 0;
  if (!bad && mx > 0.f) {
    int E;
    frexpf(mx, &E);          // mx in [2^(E-1), 2^E)
    esc = 11 - E;
    esc = esc < -120 ? -120 : (esc > 120 ? 120 : esc);
  }
  return esc;
}

// Largest magnitude of row `src` (K elements) and whether any is non-finite,
// over the whole thread block.  `sh` holds 2 * (blockDim.x / 64) ints.
template <int DT>
__device__ inline int block_row_exponent(const void* src, int K, int* sh) {
  float mx = 0.f;
  int bad = 0;
  for (int i = 4 * threadIdx.x; i < K; i += 4 * blockDim.x) {
    float v[4];
    load4_act<DT>(src, (size_t)i, v);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = fabsf(v[e]);
      bad |= !(a <= 3.402823466e38f);   // inf or NaN
      mx = fmaxf(mx, a);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    bad |= __shfl_xor(bad, o, 64);
  }
  const int nw = blockDim.x >> 6, w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    sh[w] = __float_as_int(mx);
    sh[nw + w] = bad;
  }
  __syncthreads();
  for (int i = 0; i < nw; ++i) {
    mx = fmaxf(mx, __int_as_float(sh[i]));
    bad |= sh[nw + i];
  }
  return row_exponent(mx, bad);
}

// Stage block kb of image row `row` from the row's source elements, scaled by
// 2^esc.  l = lane index within the half-wave (0..31).
template <int DT>
__device__ inline void stage_block(const void* src, int row, int kb, int esc, int layout,
                                   const XImg& img, int l) {
  const int K = img.K;
  const int k0 = kb * 256;
  float v[8];
  size_t dst;
  if (layout == XL_PERM) {
    // lane = chunk (t, g) of the block: element e = 2j + hb <-> k = 16 s + 4 hs + j + 8 hb
    const int t = l >> 2, g = l & 3, s = 4 * g + (t >> 1), hs = t & 1;
    float a[4], b[4];
    load4_act<DT>(src, k0 + 16 * s + 4 * hs, a);
    load4_act<DT>(src, k0 + 16 * s + 4 * hs + 8, b);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = a[j];
      v[2 * j + 1] = b[j];
    }
    dst = (size_t)row * K + (size_t)(kb * 32 + l) * 8;
  } else {
    const int ka = k0 + 8 * l;
    if (ka >= K) return;
    load4_act<DT>(src, ka, v);
    load4_act<DT>(src, ka + 4, v + 4);
    dst = (size_t)row * K + ka;
  }
  h8_t hv, lv;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int sh = layout == XL_PERM ? esc - 2 * (e >> 1) : esc;   // 4^-j folded in (PERM)
    _Float16 h, lo;
    split16(ldexpf(v[e], sh), h, lo);
    hv[e] = h;
    lv[e] = lo;
  }
  *(h8_t*)(img.hi + dst) = hv;
  *(h8_t*)(img.lo + dst) = lv;
  if (layout == XL_PERM && l < 16) {   // sum of sub-block l (the min term)
    float a[4], acc = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      load4_act<DT>(src, k0 + 16 * l + 4 * q, a);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc += ldexpf(a[i], esc);
    }
    _Float16 h, lo;
    split16(acc, h, lo);
    _Float16* sp = img.sx + (size_t)row * (K / 8) + (kb * 4 + (l >> 2)) * 8 + (l & 3);
    sp[0] = h;
    sp[4] = lo;
  }
}

// The whole thread block stages row `row` of src ([rows, K], row-major).
template <int DT>
__device__ inline void stage_row(const void* src, int row, int layout, const XImg& img, int* sh) {
  const int K = img.K;
  const size_t base = (size_t)row * K;
  const void* rs = DT == SV_BF16 ? (const void*)((const uint16_t*)src + base)
                                 : (const void*)((const float*)src + base);
  const int esc = block_row_exponent<DT>(rs, K, sh);
  const int nbk = (K + 255) / 256;
  for (int kb = threadIdx.x >> 5; kb < nbk; kb += blockDim.x >> 5)
    stage_block<DT>(rs, row, kb, esc, layout, img, threadIdx.x & 31);
  if (threadIdx.x == 0) img.rscale[row] = ldexpf(1.f, -esc);
}

}  // namespace sv

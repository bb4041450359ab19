// Device routines that stage activation rows into an XImg (layout and scaling
// described in sv_internal.h).  One thread block per row, 32 lanes -- half a
// wave -- per 256-element block, each lane holding 8 elements.
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

constexpr int XIMG_MAX_K = 16384;   // longest row the staging routines take

// The whole thread block (NT threads) stages row `row` of an activation
// matrix [rows, K] whose elements load4(k, v) reads (4 consecutive elements of
// the row from element k).  Every element is loaded once, into registers, with
// all loads in flight together: half-wave h takes 256-element blocks h, h + NT/32, ...
// (PERM: lane (t, g) holds elements 16 s + 4 hs + j and 16 s + 4 hs + 8 + j,
// j = 0..3, of sub-block s = 4 g + t/2, hs = t & 1; PLAIN: lane l holds
// elements 8 l .. 8 l + 7).  The row's largest magnitude is reduced over the
// block (its power-of-two scale), then each lane converts its own elements;
// a sub-block's 16-element sum is the lane's 8 plus those of lane l ^ 4.
template <int NT, class LOAD4>
__device__ inline void stage_row_l(int row, int layout, const XImg& img, int* sh, LOAD4 load4) {
  constexpr int NHW = NT / 32, MAXB = (XIMG_MAX_K / 256 + NHW - 1) / NHW;
  const int K = img.K, nbk = (K + 255) / 256;
  const int l = threadIdx.x & 31, hw = threadIdx.x >> 5;
  const bool perm = layout == XL_PERM;
  const int t = l >> 2, g = l & 3, s = 4 * g + (t >> 1), hs = t & 1;
  const size_t base = (size_t)row * K;
  float v[MAXB][8];
  float mx = 0.f;
  int bad = 0;
#pragma unroll
  for (int i = 0; i < MAXB; ++i) {
    const int kb = hw + NHW * i;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[i][e] = 0.f;
    if (kb < nbk) {
      const int k0 = kb * 256;
      if (perm) {
        float a[4], b[4];
        load4(k0 + 16 * s + 4 * hs, a);
        load4(k0 + 16 * s + 4 * hs + 8, b);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[i][2 * j] = a[j];
          v[i][2 * j + 1] = b[j];
        }
      } else if (k0 + 8 * l < K) {
        load4(k0 + 8 * l, v[i]);
        load4(k0 + 8 * l + 4, v[i] + 4);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < MAXB; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float a = fabsf(v[i][e]);
      bad |= !(a <= 3.402823466e38f);   // inf or NaN
      mx = fmaxf(mx, a);
    }
  mx = wave_allreduce(mx, [](float x, float y) { return fmaxf(x, y); });
  bad = __any(bad) ? 1 : 0;
  constexpr int NW = NT / 64;
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sh[w] = __float_as_int(mx);
    sh[NW + w] = bad;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    mx = fmaxf(mx, __int_as_float(sh[i]));
    bad |= sh[NW + i];
  }
  const int esc = row_exponent(mx, bad);
#pragma unroll
  for (int i = 0; i < MAXB; ++i) {
    const int kb = hw + NHW * i;
    if (kb >= nbk) continue;   // (uniform in the half-wave)
    const int k0 = kb * 256;
    if (!perm && k0 + 8 * l >= K) continue;
    const size_t dst = perm ? base + (size_t)(kb * 32 + l) * 8 : base + k0 + 8 * l;
    h8_t hv, lv;
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int shf = perm ? esc - 2 * (e >> 1) : esc;   // 4^-j folded in (PERM)
      _Float16 h, lo;
      split16(ldexpf(v[i][e], shf), h, lo);
      hv[e] = h;
      lv[e] = lo;
      part += ldexpf(v[i][e], esc);
    }
    *(h8_t*)(img.hi + dst) = hv;
    *(h8_t*)(img.lo + dst) = lv;
    if (perm) {   // sum of sub-block s (the min term): this lane's 8 and lane l ^ 4's
      const float sum = part + __shfl_xor(part, 4, 32);
      if (hs == 0) {
        _Float16 h, lo;
        split16(sum, h, lo);
        _Float16* sp = img.sx + (size_t)row * (K / 8) + (kb * 4 + g) * 8 + (t >> 1);
        sp[0] = h;
        sp[4] = lo;
      }
    }
  }
  if (threadIdx.x == 0) img.rscale[row] = ldexpf(1.f, -esc);
}

// Row `row` of src ([rows, K] in element type DT).
template <int DT, int NT>
__device__ inline void stage_row(const void* src, int row, int layout, const XImg& img, int* sh) {
  const size_t base = (size_t)row * img.K;
  const void* rs = DT == SV_BF16 ? (const void*)((const uint16_t*)src + base)
                                 : (const void*)((const float*)src + base);
  stage_row_l<NT>(row, layout, img, sh, [&](int k, float* v) { load4_act<DT>(rs, k, v); });
}

}  // namespace sv

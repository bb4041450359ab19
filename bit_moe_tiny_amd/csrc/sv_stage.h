// Device routine that stages one 256-element block of an activation row into
// an XImg (layout and scaling described in sv_internal.h).  32 lanes -- half a
// wave -- share one block: each lane converts 8 elements, the block's scale
// comes from a 32-lane max, so a whole row set is staged in one parallel pass.
#pragma once

#include "sv_internal.h"

namespace sv {

template <int DT>
__device__ inline void load4_act(const void* src, size_t idx, float* v) {
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

__device__ inline void split16(float v, _Float16& hi, _Float16& lo) {
  hi = (_Float16)v;
  lo = (_Float16)(v - (float)hi);
}

// Stage block kb of image row `row`, whose source elements start at
// src[src_base].  l = lane index within the half-wave (0..31).
template <int DT>
__device__ inline void stage_block(const void* src, size_t src_base, int row, int kb, int layout,
                                   const XImg& img, int l) {
  const int K = img.K;
  const int k0 = kb * 256;
  float v[8];
  size_t dst;
  if (layout == XL_PERM) {
    // lane = chunk (t, g) of the block: element e = 2j + hb <-> k = 16 s + 4 hs + j + 8 hb
    const int t = l >> 2, g = l & 3, s = 4 * g + (t >> 1), hs = t & 1;
    float a[4], b[4];
    load4_act<DT>(src, src_base + k0 + 16 * s + 4 * hs, a);
    load4_act<DT>(src, src_base + k0 + 16 * s + 4 * hs + 8, b);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = a[j];
      v[2 * j + 1] = b[j];
    }
    dst = (size_t)row * K + (size_t)(kb * 32 + l) * 8;
  } else {
    const int ka = k0 + 8 * l;
    if (ka < K) {
      load4_act<DT>(src, src_base + ka, v);
      load4_act<DT>(src, src_base + ka + 4, v + 4);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = 0.f;
    }
    dst = (size_t)row * K + ka;
  }
  float mx = 0.f;
  int bad = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float a = fabsf(v[e]);
    bad |= !(a <= 3.402823466e38f);   // inf or NaN
    mx = fmaxf(mx, a);
  }
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) {
    mx = fmaxf(mx, __shfl_xor(mx, o, 32));
    bad |= __shfl_xor(bad, o, 32);
  }
  int esc = 0;
  if (!bad && mx > 0.f) {
    int E;
    frexpf(mx, &E);          // mx in [2^(E-1), 2^E)
    esc = 11 - E;            // block max lands in [2^10, 2^11)
    esc = esc < -120 ? -120 : (esc > 120 ? 120 : esc);
  }
  if (layout == XL_PLAIN && k0 + 8 * l >= K) return;
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
      load4_act<DT>(src, src_base + k0 + 16 * l + 4 * q, a);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc += ldexpf(a[i], esc);
    }
    _Float16 h, lo;
    split16(acc, h, lo);
    const size_t so = (size_t)row * (K / 16) + kb * 16 + l;
    img.sxh[so] = h;
    img.sxl[so] = lo;
  }
  if (l == 0) img.bscale[(size_t)row * img.nbk + kb] = ldexpf(1.f, -esc);
}

// Stage rows [0, n_rows) of `src` ([rows, K], row-major) with one half-wave per
// (row, block); `gid` enumerates (row, block) pairs.
template <int DT>
__device__ inline void stage_gid(const void* src, int n_rows, int layout, const XImg& img, int gid,
                                 int l) {
  const int row = gid / img.nbk, kb = gid - row * img.nbk;
  if (row >= n_rows) return;
  stage_block<DT>(src, (size_t)row * img.K, row, kb, layout, img, l);
}

}  // namespace sv

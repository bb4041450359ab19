// Device routine that stages one activation row into an XImg (see stage.hip).
#pragma once

#include "sv_internal.h"

namespace sv {

__device__ inline float load_act(const void* src, int dtype, size_t idx) {
  if (dtype == SV_BF16) {
    uint32_t b = ((const uint16_t*)src)[idx];
    return __uint_as_float(b << 16);
  }
  return ((const float*)src)[idx];
}

__device__ inline float wave_max_f(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ inline int wave_or_i(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v |= __shfl_xor(v, o, 64);
  return v;
}

__device__ inline void split16(float v, _Float16& hi, _Float16& lo) {
  hi = (_Float16)v;
  lo = (_Float16)(v - (float)hi);
}

// Stage source row `src[base .. base+K)` into image row `row`.  256 threads;
// `xs` is K floats of LDS, `red`/`flag` 4 entries each.
__device__ inline void stage_row(const void* src, int dtype, size_t base, int row, int K,
                                 int layout, XImg img, float* xs, float* red, int* flag) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  float mx = 0.f;
  int bad = 0;
  for (int k = tid; k < K; k += 256) {
    float v = load_act(src, dtype, base + k);
    xs[k] = v;
    float a = fabsf(v);
    bad |= !(a <= 3.402823466e38f);   // inf or NaN
    mx = fmaxf(mx, a);
  }
  mx = wave_max_f(mx);
  bad = wave_or_i(bad);
  if (lane == 0) {
    red[wv] = mx;
    flag[wv] = bad;
  }
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  bad = flag[0] | flag[1] | flag[2] | flag[3];
  int esc = 0;
  if (!bad && mx > 0.f) {
    int E;
    frexpf(mx, &E);          // mx in [2^(E-1), 2^E)
    esc = 11 - E;            // mx * 2^esc in [2^10, 2^11)
    esc = esc < -120 ? -120 : (esc > 120 ? 120 : esc);
  }
  const size_t rb = (size_t)row * K;
  if (layout == XL_PERM) {
    // chunk = 8 halves read by one lane for one matrix-core step:
    // ch = (kb*8 + t)*4 + g; element e = 2j + hb <-> k = kb*256 + 16*s + 4*hs + j + 8*hb,
    // s = 4g + (t>>1), hs = t&1, scaled by 4^-j.
    for (int ch = tid; ch < K / 8; ch += 256) {
      const int kb = ch >> 5, t = (ch >> 2) & 7, g = ch & 3;
      const int s = 4 * g + (t >> 1), hs = t & 1;
      h8_t hv, lv;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = e >> 1, hb = e & 1;
        const int k = kb * 256 + 16 * s + 4 * hs + j + 8 * hb;
        _Float16 h, l;
        split16(ldexpf(xs[k], esc - 2 * j), h, l);
        hv[e] = h;
        lv[e] = l;
      }
      *(h8_t*)(img.hi + rb + (size_t)ch * 8) = hv;
      *(h8_t*)(img.lo + rb + (size_t)ch * 8) = lv;
    }
    const size_t sb0 = (size_t)row * (K / 16);
    for (int sb = tid; sb < K / 16; sb += 256) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc += ldexpf(xs[16 * sb + i], esc);
      _Float16 h, l;
      split16(acc, h, l);
      img.sxh[sb0 + sb] = h;
      img.sxl[sb0 + sb] = l;
    }
  } else {
    for (int k = tid; k < K; k += 256) {
      _Float16 h, l;
      split16(ldexpf(xs[k], esc), h, l);
      img.hi[rb + k] = h;
      img.lo[rb + k] = l;
    }
  }
  if (tid == 0) img.rscale[row] = ldexpf(1.f, -esc);
}

}  // namespace sv

// Two-bit block x activation-image contraction on the fp16 matrix cores.
//
// One wave computes a 16 (weight rows n) x 16 (activation columns c) tile over
// a range of 256-element blocks with v_mfma_f32_16x16x32_f16:
//   A operand = activation image (lane: column c = lane&15, k-group g = lane>>4)
//   B operand = weights          (lane: row n = lane&15,    k-group g = lane>>4)
//   result    = D[c][n]: lane holds n = lane&15 and c = 4*(lane>>4) + 0..3.
// Each lane loads, per block, the 16 code bytes of sub-blocks 4g..4g+3 of its
// row (one dwordx4), their 4 nibble bytes (one dword) and the row's d / dmin.
// Per step t (0..7) it turns one half of one sub-block into 8 fp16 weights
// sc * q * 4^j -- exact integers: the code is OR-ed into the mantissa of
// 1024.0 at bit position 2j (value 1024 + 4^j q) and one packed fma with
// (sc, -1024 sc) removes the offset and applies the sub-block scale.  The
// image carries the matching 4^-j.  The block's min term dmin * m * sum(x)
// is one 16x16x16 product of the per-sub-block sums with the m nibbles, and
// the block scales are applied in fp32:  acc += d * D_codes - dmin * D_min.
#pragma once

#include "sv_internal.h"

namespace sv {

__device__ inline float f16bits_to_f32(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

__device__ inline h2_t as_h2(uint32_t v) { return __builtin_bit_cast(h2_t, v); }

struct XRow {
  const _Float16* hi;   // image row (nullptr: padding column, contributes zero)
  const _Float16* lo;
  const _Float16* sxh;
  const _Float16* sxl;
};

__device__ inline XRow xrow(const XImg& img, int row) {
  XRow r;
  if (row < 0) {
    r.hi = r.lo = r.sxh = r.sxl = nullptr;
  } else {
    r.hi = img.hi + (size_t)row * img.K;
    r.lo = img.lo + (size_t)row * img.K;
    r.sxh = img.sxh + (size_t)row * (img.K / 16);
    r.sxl = img.sxl + (size_t)row * (img.K / 16);
  }
  return r;
}

struct Q2Blk {
  uint4 qs;
  uint32_t sc;
  uint16_t d, dm;
};

__device__ inline Q2Blk q2_load(const Q2View& W, int n, int kb, int g) {
  const size_t b = (size_t)n * W.nb + kb;
  Q2Blk k;
  k.qs = *(const uint4*)(W.qs + b * 64 + 16 * g);
  k.sc = *(const uint32_t*)(W.sc + b * 16 + 4 * g);
  k.d = W.d[b];
  k.dm = W.dm[b];
  return k;
}

// Weights of step t as the B operand (8 fp16).
__device__ inline h8_t q2_bop(const Q2Blk& k, int t) {
  const int i = t >> 1, hs = t & 1;
  const uint32_t dw = (i == 0 ? k.qs.x : i == 1 ? k.qs.y : i == 2 ? k.qs.z : k.qs.w) >> (8 * hs);
  const float scf = (float)((k.sc >> (8 * i)) & 15u);
  const _Float16 sch = (_Float16)scf;
  const _Float16 negh = (_Float16)(-1024.f * scf);
  const h2_t scp = {sch, sch};
  const h2_t neg = {negh, negh};
  h8_t b;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const h2_t p = as_h2((dw & (0x00030003u << (2 * j))) | 0x64006400u);
    const h2_t a = __builtin_elementwise_fma(p, scp, neg);
    b[2 * j] = a.x;
    b[2 * j + 1] = a.y;
  }
  return b;
}

// m nibbles of sub-blocks 4g..4g+3 as the B operand of the min-term product.
__device__ inline h4_t q2_mop(const Q2Blk& k) {
  h4_t m;
#pragma unroll
  for (int i = 0; i < 4; ++i) m[i] = (_Float16)(float)((k.sc >> (8 * i + 4)) & 15u);
  return m;
}

__device__ inline h8_t ld_h8(const _Float16* p) { return *(const h8_t*)p; }
__device__ inline h4_t ld_h4(const _Float16* p) { return *(const h4_t*)p; }

// Accumulate block kb of weight row n (this lane's row) against the image row
// of this lane's column.  acc: the lane's 4 outputs D[4g+e][n].
template <bool USE_LO>
__device__ inline void q2_block(const Q2Blk& k, const XRow& x, int kb, int g, f4_t& acc) {
  const f4_t zero = {0.f, 0.f, 0.f, 0.f};
  const h8_t z8 = {0, 0, 0, 0, 0, 0, 0, 0};
  const h4_t z4 = {0, 0, 0, 0};
  f4_t dt = zero;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const h8_t b = q2_bop(k, t);
    const size_t off = (size_t)((kb * 8 + t) * 4 + g) * 8;
    const h8_t a = x.hi ? ld_h8(x.hi + off) : z8;
    dt = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, dt, 0, 0, 0);
    if (USE_LO) {
      const h8_t al = x.lo ? ld_h8(x.lo + off) : z8;
      dt = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, b, dt, 0, 0, 0);
    }
  }
  const h4_t m = q2_mop(k);
  const size_t so = (size_t)kb * 16 + 4 * g;
  const h4_t sx = x.sxh ? ld_h4(x.sxh + so) : z4;
  // the 16-element sums are never fp16-exact: their remainder is always used
  const h4_t sxl = x.sxl ? ld_h4(x.sxl + so) : z4;
  f4_t dm = __builtin_amdgcn_mfma_f32_16x16x16f16(sx, m, zero, 0, 0, 0);
  dm = __builtin_amdgcn_mfma_f32_16x16x16f16(sxl, m, dm, 0, 0, 0);
  const float d = f16bits_to_f32(k.d), dmin = f16bits_to_f32(k.dm);
#pragma unroll
  for (int e = 0; e < 4; ++e) acc[e] = fmaf(d, dt[e], fmaf(-dmin, dm[e], acc[e]));
}

}  // namespace sv

// Two-bit block x activation-image contraction on the fp16 matrix cores.
//
// One wave computes a 16 (weight rows n) x 16 (activation columns c) tile over
// a range of 256-element blocks with v_mfma_f32_16x16x32_f16:
//   A operand = activation image (lane: column c = lane&15, k-group g = lane>>4)
//   B operand = weights          (lane: row n = lane&15,    k-group g = lane>>4)
//   result    = D[c][n]: lane holds n = lane&15 and c = 4*(lane>>4) + 0..3.
// Each lane loads, per block, the 16 code bytes of sub-blocks 4g..4g+3 of its
// row (one dwordx4), their 4 nibble bytes (one dword) and the row's d / dmin;
// a wave issues these loads for up to 8 blocks before computing any of them.
// Per step t (0..7) a lane turns one half of one sub-block into 8 fp16 weights
// sc * q * 4^j -- exact integers: the code is OR-ed into the mantissa of
// 1024.0 at bit position 2j (value 1024 + 4^j q) and one packed fma with
// (sc, -1024 sc) removes the offset and applies the sub-block scale.  The
// image carries the matching 4^-j.  The block's min term dmin * m * sum(x)
// is one 16x16x16 product of the per-sub-block sums with the m nibbles, and
// the block scales are applied in fp32:
//   acc += s_x * (d * D_codes - dmin * D_min),  s_x = the image's block scale.
#pragma once

#include "sv_internal.h"

namespace sv {

__device__ inline float f16bits_to_f32(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

__device__ inline h2_t as_h2(uint32_t v) { return __builtin_bit_cast(h2_t, v); }

struct XRow {
  const _Float16* hi;   // image row of this lane's column
  const _Float16* lo;
  const _Float16* sxh;
  const _Float16* sxl;
  const float* bs;      // block scales of the row
};

// `row` is this lane's column; padding columns (beyond the rows in use) read
// row `fallback` instead: an output column depends only on its own operand
// row, and padding columns are never stored, so their values do not matter --
// this keeps every load unconditional (no branches, no serialising waits).
__device__ inline XRow xrow(const XImg& img, int row, int fallback) {
  const size_t r = (size_t)(row >= 0 ? row : fallback);
  XRow x;
  x.hi = img.hi + r * img.K;
  x.lo = img.lo + r * img.K;
  x.sxh = img.sxh + r * (img.K / 16);
  x.sxl = img.sxl + r * (img.K / 16);
  x.bs = img.bscale + r * img.nbk;
  return x;
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

// (x & m) | o in one instruction.  gfx9 VOP3 encodings take no 32-bit
// literals, so the compiler splits this into v_and_b32 + v_or_b32 with
// literals; here the mask comes in an SGPR and the OR constant in a VGPR.
__device__ inline uint32_t and_or(uint32_t x, uint32_t m, uint32_t o) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(m), "v"(o));
  return r;
}

// fp16 (1024 + byte) pairs from bytes (0,1) / (2,3) of u: v_perm_b32 picks
// bytes 0-3 from its second operand and 4-7 from its first.
__device__ inline h2_t q2_bytes01(uint32_t u) {
  return __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u));
}
__device__ inline h2_t q2_bytes23(uint32_t u) {
  return __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u));
}

// Per-block constants of a lane: the scales of its 4 sub-blocks as fp16
// pairs (sc_i, sc_{i+1}) and (-1024 sc_i, ...), and the 4 mins as an fp16
// vector -- from the nibble dword in a handful of packed operations.
struct Q2Sc {
  h2_t sc01, sc23, ng01, ng23;
  h4_t m;
};

__device__ inline Q2Sc q2_scales(uint32_t scw) {
  const h2_t k1024 = {(_Float16)1024.f, (_Float16)1024.f};
  const h2_t kneg = {(_Float16)-1024.f, (_Float16)-1024.f};
  const uint32_t lo = scw & 0x0F0F0F0Fu, hi = (scw >> 4) & 0x0F0F0F0Fu;
  Q2Sc r;
  r.sc01 = q2_bytes01(lo) - k1024;   // exact small integers
  r.sc23 = q2_bytes23(lo) - k1024;
  r.ng01 = r.sc01 * kneg;
  r.ng23 = r.sc23 * kneg;
  const h2_t m01 = q2_bytes01(hi) - k1024, m23 = q2_bytes23(hi) - k1024;
  r.m = (h4_t){m01.x, m01.y, m23.x, m23.y};
  return r;
}

// Weights of step t as the B operand (8 fp16): 4^j * sc * q for the 8 codes.
// `magic` holds 0x64006400 (fp16 pair 1024.0) in a register.
__device__ inline h8_t q2_bop(const uint4& qs, const Q2Sc& S, int t, uint32_t magic) {
  const int i = t >> 1, hs = t & 1;
  const uint32_t dw = (i == 0 ? qs.x : i == 1 ? qs.y : i == 2 ? qs.z : qs.w) >> (8 * hs);
  const h2_t scp = (i == 0) ? (h2_t){S.sc01.x, S.sc01.x} : (i == 1) ? (h2_t){S.sc01.y, S.sc01.y}
                 : (i == 2) ? (h2_t){S.sc23.x, S.sc23.x} : (h2_t){S.sc23.y, S.sc23.y};
  const h2_t neg = (i == 0) ? (h2_t){S.ng01.x, S.ng01.x} : (i == 1) ? (h2_t){S.ng01.y, S.ng01.y}
                 : (i == 2) ? (h2_t){S.ng23.x, S.ng23.x} : (h2_t){S.ng23.y, S.ng23.y};
  h8_t b;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const h2_t p = as_h2(and_or(dw, 0x00030003u << (2 * j), magic));
    const h2_t a = __builtin_elementwise_fma(p, scp, neg);
    b[2 * j] = a.x;
    b[2 * j + 1] = a.y;
  }
  return b;
}

// The OR constant as an opaque register value (kept in one VGPR).
__device__ inline uint32_t q2_magic() {
  uint32_t m = 0x64006400u;
  asm volatile("" : "+v"(m));
  return m;
}

// Activation operands of one block for this lane's column.
template <bool USE_LO>
struct XBlk {
  h8_t hi[8];
  h8_t lo[USE_LO ? 8 : 1];
  h4_t sxh, sxl;
  f4_t xs;   // block scales of the lane's 4 output columns
};

template <bool USE_LO>
__device__ inline void x_load(const XRow& x, int kb, int lane, XBlk<USE_LO>& X) {
  const int g = lane >> 4;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const size_t off = (size_t)((kb * 8 + t) * 4 + g) * 8;
    X.hi[t] = *(const h8_t*)(x.hi + off);
    if (USE_LO) X.lo[t] = *(const h8_t*)(x.lo + off);
  }
  const size_t so = (size_t)kb * 16 + 4 * g;
  X.sxh = *(const h4_t*)(x.sxh + so);
  X.sxl = *(const h4_t*)(x.sxl + so);
  // lane c (< 16) holds column c's A operand: fetch the 4 output columns' scales from there
  const float s_own = x.bs[kb];
#pragma unroll
  for (int e = 0; e < 4; ++e) X.xs[e] = __shfl(s_own, 4 * g + e, 64);
}

// acc (the lane's 4 outputs D[4g+e][n]) += block contribution.
template <bool USE_LO>
__device__ inline void q2_block(const Q2Blk& k, const XBlk<USE_LO>& X, f4_t& acc) {
  const f4_t zero = {0.f, 0.f, 0.f, 0.f};
  const uint32_t magic = q2_magic();
  const Q2Sc S = q2_scales(k.sc);
  f4_t dt = zero;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const h8_t b = q2_bop(k.qs, S, t, magic);
    dt = __builtin_amdgcn_mfma_f32_16x16x32_f16(X.hi[t], b, dt, 0, 0, 0);
    if (USE_LO) dt = __builtin_amdgcn_mfma_f32_16x16x32_f16(X.lo[USE_LO ? t : 0], b, dt, 0, 0, 0);
  }
  // the 16-element sums are never fp16-exact: their remainder is always used
  f4_t dm = __builtin_amdgcn_mfma_f32_16x16x16f16(X.sxh, S.m, zero, 0, 0, 0);
  dm = __builtin_amdgcn_mfma_f32_16x16x16f16(X.sxl, S.m, dm, 0, 0, 0);
  const float d = f16bits_to_f32(k.d), dmin = f16bits_to_f32(k.dm);
#pragma unroll
  for (int e = 0; e < 4; ++e) acc[e] = fmaf(X.xs[e], fmaf(d, dt[e], -dmin * dm[e]), acc[e]);
}

// One pipeline slot: a block's weights for NM matrices and its activation operands.
template <int NM, bool USE_LO>
struct Q2Slot {
  Q2Blk w[NM];
  XBlk<USE_LO> x;
};

template <int NM, bool USE_LO>
__device__ inline void q2_slot_load(const Q2View* W, int n, int kb, const XRow& x, int lane,
                                    Q2Slot<NM, USE_LO>& S) {
  x_load<USE_LO>(x, kb, lane, S.x);
#pragma unroll
  for (int m = 0; m < NM; ++m) S.w[m] = q2_load(W[m], n, kb, lane >> 4);
}

// NM matrices (sharing one activation row per lane) over NB blocks from kb0
// of weight row n, software-pipelined over three register slots: the weights
// and activation operands of block i+2 are requested before block i is
// computed (i+1 with the remainder operand, whose registers allow only two
// slots).  Vector-memory loads retire in issue order, so they are issued in
// the order they are used and without branches; the wait for block i then
// leaves the later blocks in flight.  The slots are distinct variables (not an
// array) so each keeps its own registers, and a scheduling barrier keeps every
// block's loads in its stage.
template <int NM, bool USE_LO, int NB>
__device__ inline void q2_pipe(const Q2View* W, int n, int kb0, const XRow& x, int lane,
                               f4_t* acc) {
  constexpr int PD = USE_LO ? 1 : 2;
  Q2Slot<NM, USE_LO> s0, s1, s2;
  q2_slot_load<NM, USE_LO>(W, n, kb0, x, lane, s0);
  if (PD > 1 && NB > 1) q2_slot_load<NM, USE_LO>(W, n, kb0 + 1, x, lane, s1);
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int ld = i + PD;   // block requested in this stage
    if (ld < NB) {
      const int sl = ld % (PD + 1);
      q2_slot_load<NM, USE_LO>(W, n, kb0 + ld, x, lane, sl == 0 ? s0 : sl == 1 ? s1 : s2);
    }
    const int sc = i % (PD + 1);
    const Q2Slot<NM, USE_LO>& cur = sc == 0 ? s0 : sc == 1 ? s1 : s2;
#pragma unroll
    for (int m = 0; m < NM; ++m) q2_block<USE_LO>(cur.w[m], cur.x, acc[m]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Any block count: pipelined chunks of 8, then the remainder.
template <int NM, bool USE_LO>
__device__ inline void q2_run(const Q2View* W, int n, int kb0, int nblk, const XRow& x, int lane,
                              f4_t* acc) {
  int kb = kb0;
  for (; kb + 8 <= kb0 + nblk; kb += 8) q2_pipe<NM, USE_LO, 8>(W, n, kb, x, lane, acc);
  switch (kb0 + nblk - kb) {
    case 1: q2_pipe<NM, USE_LO, 1>(W, n, kb, x, lane, acc); break;
    case 2: q2_pipe<NM, USE_LO, 2>(W, n, kb, x, lane, acc); break;
    case 3: q2_pipe<NM, USE_LO, 3>(W, n, kb, x, lane, acc); break;
    case 4: q2_pipe<NM, USE_LO, 4>(W, n, kb, x, lane, acc); break;
    case 5: q2_pipe<NM, USE_LO, 5>(W, n, kb, x, lane, acc); break;
    case 6: q2_pipe<NM, USE_LO, 6>(W, n, kb, x, lane, acc); break;
    case 7: q2_pipe<NM, USE_LO, 7>(W, n, kb, x, lane, acc); break;
    default: break;
  }
}

// ---------------------------------------------------------------------------
// Variant with the activation operands in LDS.  Used where the waves of a
// block share their activation rows: the rows are staged once per block, the
// per-step operand reads go to LDS (their waits are counted apart from the
// weight loads, which stay in flight), and the registers hold only weights.
struct XLds {
  const _Float16* hi;    // [4][K] PERM layout
  const _Float16* lo;
  const _Float16* sxh;   // [4][K/16]
  const _Float16* sxl;
  const float* bs;       // [4][nbk]
  int K, nbk;
};

// acc += block kb of weight row n against LDS column `col` (0..3) of this lane.
__device__ inline void q2_block_lds(const Q2Blk& k, const XLds& X, int col, int kb, int lane,
                                    f4_t& acc) {
  const int g = lane >> 4;
  const f4_t zero = {0.f, 0.f, 0.f, 0.f};
  const _Float16* xh = X.hi + (size_t)col * X.K;
  const _Float16* xl = X.lo + (size_t)col * X.K;
  const uint32_t magic = q2_magic();
  const Q2Sc S = q2_scales(k.sc);
  f4_t dt = zero;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const h8_t b = q2_bop(k.qs, S, t, magic);
    const int off = ((kb * 8 + t) * 4 + g) * 8;
    dt = __builtin_amdgcn_mfma_f32_16x16x32_f16(*(const h8_t*)(xh + off), b, dt, 0, 0, 0);
    dt = __builtin_amdgcn_mfma_f32_16x16x32_f16(*(const h8_t*)(xl + off), b, dt, 0, 0, 0);
  }
  const int so = col * (X.K / 16) + kb * 16 + 4 * g;
  f4_t dm = __builtin_amdgcn_mfma_f32_16x16x16f16(*(const h4_t*)(X.sxh + so), S.m, zero, 0, 0, 0);
  dm = __builtin_amdgcn_mfma_f32_16x16x16f16(*(const h4_t*)(X.sxl + so), S.m, dm, 0, 0, 0);
  const float d = f16bits_to_f32(k.d), dmin = f16bits_to_f32(k.dm);
  // block scales of the lane's 4 output columns (column c of the tile = LDS row c & 3)
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float xs = X.bs[((4 * g + e) & 3) * X.nbk + kb];
    acc[e] = fmaf(xs, fmaf(d, dt[e], -dmin * dm[e]), acc[e]);
  }
}

// NB blocks from kb0, weights pipelined PD = 3 blocks ahead in registers.
template <int NB>
__device__ inline void q2_pipe_lds(const Q2View& W, int n, int kb0, const XLds& X, int col,
                                   int lane, f4_t& acc) {
  constexpr int PD = 3;
  const int g = lane >> 4;
  Q2Blk s0, s1, s2, s3;
  s0 = q2_load(W, n, kb0, g);
  if (NB > 1) s1 = q2_load(W, n, kb0 + 1, g);
  if (NB > 2) s2 = q2_load(W, n, kb0 + 2, g);
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int ld = i + PD;
    if (ld < NB) {
      const int sl = ld & 3;
      (sl == 0 ? s0 : sl == 1 ? s1 : sl == 2 ? s2 : s3) = q2_load(W, n, kb0 + ld, g);
    }
    const int sc = i & 3;
    q2_block_lds(sc == 0 ? s0 : sc == 1 ? s1 : sc == 2 ? s2 : s3, X, col, kb0 + i, lane, acc);
    __builtin_amdgcn_sched_barrier(0);
  }
}

__device__ inline void q2_run_lds(const Q2View& W, int n, int nblk, const XLds& X, int col,
                                  int lane, f4_t& acc) {
  int kb = 0;
  for (; kb + 8 <= nblk; kb += 8) q2_pipe_lds<8>(W, n, kb, X, col, lane, acc);
  switch (nblk - kb) {
    case 1: q2_pipe_lds<1>(W, n, kb, X, col, lane, acc); break;
    case 2: q2_pipe_lds<2>(W, n, kb, X, col, lane, acc); break;
    case 3: q2_pipe_lds<3>(W, n, kb, X, col, lane, acc); break;
    case 4: q2_pipe_lds<4>(W, n, kb, X, col, lane, acc); break;
    case 5: q2_pipe_lds<5>(W, n, kb, X, col, lane, acc); break;
    case 6: q2_pipe_lds<6>(W, n, kb, X, col, lane, acc); break;
    case 7: q2_pipe_lds<7>(W, n, kb, X, col, lane, acc); break;
    default: break;
  }
}

}  // namespace sv

// Two-bit block x activation contraction on the fp16 matrix cores, with the
// activation rows held in LDS.
//
// One wave computes a 16 (weight rows n) x 16 (activation columns c) tile over
// a range of 256-element blocks of one matrix with v_mfma_f32_16x16x32_f16:
//   A operand = activations (lane: column c = lane&15, k-group g = lane>>4),
//               read from the block's LDS copy of the rows;
//   B operand = weights (lane: row n = lane&15, k-group g = lane>>4);
//   result    = D[c][n]: lane holds n = lane&15 and c = 4*(lane>>4) + 0..3.
//
// Weight loads are all 16 bytes per lane (the vector-memory address path, not
// HBM, limits narrower loads):
//   codes  one load per block: lane (n, g) gets the 16 code bytes of sub-blocks
//          4g..4g+3 of row n (the 4 lanes of a row cover its 64 bytes);
//   scales one load per 4 blocks: lane-row g gets all 16 nibble bytes of block
//          kb+g; two permlane16 and two permlane32 swaps transpose the 4x4
//          dwords so that every lane holds its own 4 sub-blocks of each block;
//   d/dmin one load per 8 blocks (when the row's block count is even and at
//          least 8): even lane-rows read 8 block scales d, odd lane-rows the 8
//          min-scales; one permlane16 swap per dword gives every lane both.
// All loads of a chunk of up to 8 blocks are issued before any is used, in the
// order they are consumed, so the whole chunk is in flight at once.
//
// Per block, a lane turns one half of one sub-block into 8 fp16 weights
// sc * q * 4^j per step (t = 0..7) -- exact integers: the code is OR-ed into
// the mantissa of 1024.0 at bit position 2j (value 1024 + 4^j q) and one
// packed fma with (sc, -1024 sc) removes the offset and applies the sub-block
// scale; the activation rows carry the matching 4^-j.  The min term
// dmin * m * sum(x) is one 16x16x16 product of the per-sub-block sums with the
// m nibbles.  Block scales are applied in fp32:
//   acc += s_x * (d * D_codes - dmin * D_min),  s_x = the rows' block scale.
#pragma once

#include "sv_internal.h"

namespace sv {

__device__ __forceinline__ float f16bits_to_f32(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

__device__ __forceinline__ h2_t as_h2(uint32_t v) { return __builtin_bit_cast(h2_t, v); }

// (x & m) | o in one instruction (v_and_or_b32).  gfx9 VOP3 encodings take
// no 32-bit literals, so with constant m and o the compiler would split this
// into v_and_b32 + v_or_b32; given m in an SGPR and o in a VGPR it selects the
// single instruction by itself (and, unlike inline asm, still knows which
// registers it writes, so it adds no defensive wait states).
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t o) { return (x & m) | o; }

// Constant c held in a scalar register (opaque to constant folding; not
// volatile, so that the copies are shared and hoisted out of loops).
__device__ __forceinline__ uint32_t sreg(uint32_t c) {
  asm("" : "+s"(c));
  return c;
}

// fp16 (1024 + byte) pairs from bytes (0,1) / (2,3) of u: v_perm_b32 picks
// bytes 0-3 from its second operand and 4-7 from its first.
__device__ __forceinline__ h2_t q2_bytes01(uint32_t u) {
  return __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u));
}
__device__ __forceinline__ h2_t q2_bytes23(uint32_t u) {
  return __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u));
}

// Per-block constants of a lane: the scales of its 4 sub-blocks as fp16
// pairs (sc_i, sc_{i+1}) and (-1024 sc_i, ...), and the 4 mins as an fp16
// vector -- from the nibble dword in a handful of packed operations.
struct Q2Sc {
  h2_t sc01, sc23, ng01, ng23;
  h4_t m;
};

__device__ __forceinline__ Q2Sc q2_scales(uint32_t scw) {
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
__device__ __forceinline__ h8_t q2_bop(const uint4& qs, const Q2Sc& S, int t, uint32_t magic) {
  const int i = t >> 1, hs = t & 1;
  const uint32_t dw = (i == 0 ? qs.x : i == 1 ? qs.y : i == 2 ? qs.z : qs.w) >> (8 * hs);
  const h2_t scp = (i == 0) ? (h2_t){S.sc01.x, S.sc01.x} : (i == 1) ? (h2_t){S.sc01.y, S.sc01.y}
                 : (i == 2) ? (h2_t){S.sc23.x, S.sc23.x} : (h2_t){S.sc23.y, S.sc23.y};
  const h2_t neg = (i == 0) ? (h2_t){S.ng01.x, S.ng01.x} : (i == 1) ? (h2_t){S.ng01.y, S.ng01.y}
                 : (i == 2) ? (h2_t){S.ng23.x, S.ng23.x} : (h2_t){S.ng23.y, S.ng23.y};
  h8_t b;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const h2_t p = as_h2(and_or(dw, sreg(0x00030003u << (2 * j)), magic));
    const h2_t a = __builtin_elementwise_fma(p, scp, neg);
    b[2 * j] = a.x;
    b[2 * j + 1] = a.y;
  }
  return b;
}

// The OR constant as an opaque register value (kept in one VGPR).
__device__ __forceinline__ uint32_t q2_magic() {
  uint32_t m = 0x64006400u;
  asm volatile("" : "+v"(m));
  return m;
}

// ------------------------------------------------------------ LDS rows
// Activation rows of one block in LDS (layout written by the stagers):
//   hi, lo  [ncols][rs] fp16 in the PERM order of sv_internal.h (element
//           ((kb*8 + t)*4 + g)*8 + i of a row is the A-operand value i of
//           lane-group g at step t of block kb); rs = K + 8 (16 bytes of
//           padding move each row to other banks)
//   sx      [ncols][K/8] fp16: per 4-sub-block group (kb*4 + g), the 4
//           sub-block sums' high parts then their 4 remainders
//   rsc     [16] fp32: the row scale 2^-e of column c (0 beyond ncols)
// A lane reads its column's row from a base address fixed for the chunk, so
// every read of a block is base + an immediate offset.
constexpr int XL_MAX_COLS = 8;

struct XL {
  const _Float16* hi;
  const _Float16* lo;
  const _Float16* sx;
  const float* rsc;
  int rs, sxs;
};

__host__ __device__ inline int xl_rs(int K) { return K + 8; }

__host__ __device__ inline size_t up16(size_t n) { return (n + 15) & ~size_t(15); }

__host__ __device__ inline size_t xl_bytes(int ncols, int K, bool use_lo) {
  const size_t rows = (size_t)ncols * xl_rs(K) * 2 * (use_lo ? 2 : 1);
  const size_t sx = (size_t)ncols * (K / 8) * 2;
  return up16(rows) + up16(sx) + 16 * 4;
}

template <typename P>
__device__ __forceinline__ void xl_carve(P* base, int ncols, int K, bool use_lo, P*& hi, P*& lo,
                                         P*& sx, float*& rsc) {
  uint8_t* p = (uint8_t*)base;
  const size_t row = (size_t)xl_rs(K) * 2;
  hi = (P*)p;
  lo = (P*)(p + (size_t)ncols * row);
  p += up16((size_t)ncols * row * (use_lo ? 2 : 1));
  sx = (P*)p;
  p += up16((size_t)ncols * (K / 8) * 2);
  rsc = (float*)p;
}

// ------------------------------------------------------------ wide loads
constexpr int WB = 8;   // blocks per load chunk

template <int NBW, bool WIDE_D>
struct Q2Chunk {
  uint4 qs[NBW];
  uint4 sc[(NBW + 3) / 4];
  uint4 dd;                          // WIDE_D
  uint16_t d[WIDE_D ? 1 : NBW], dm[WIDE_D ? 1 : NBW];
};

// First block of the 8-block d/dmin window of a chunk starting at kb0: even
// (so the 16-byte load is dword aligned) and inside the row; it covers 8
// blocks from an even kb0 and 7 from an odd one (chunks are cut to fit).
__device__ __forceinline__ int q2_dwin(int kb0, int nb) { return min(kb0 & ~1, nb - 8); }

// Issue every load of blocks kb0..kb0+NBW-1 of weight row n, in the order the
// blocks consume them.
template <int NBW, bool WIDE_D>
__device__ __forceinline__ void q2_chunk_load(const Q2View& W, int n, int kb0, int g,
                                     Q2Chunk<NBW, WIDE_D>& c) {
  const size_t rb = (size_t)n * W.nb;
#pragma unroll
  for (int i = 0; i < NBW; ++i) {
    if (i % 4 == 0) {
      const int kb = min(kb0 + i + g, W.nb - 1);   // lane-row g: all nibbles of block kb0+i+g
      c.sc[i / 4] = *(const uint4*)(W.sc + (rb + kb) * 16);
    }
    if (i == 0) {
      if (WIDE_D) {
        const uint16_t* pl = (g & 1) ? W.dm : W.d;
        c.dd = *(const uint4*)(pl + rb + q2_dwin(kb0, W.nb));
      }
    }
    c.qs[i] = *(const uint4*)(W.qs + (rb + kb0 + i) * 64 + 16 * g);
    if (!WIDE_D) {
      c.d[WIDE_D ? 0 : i] = W.d[rb + kb0 + i];
      c.dm[WIDE_D ? 0 : i] = W.dm[rb + kb0 + i];
    }
  }
}

// 4x4 dword transpose across the four 16-lane rows: on entry lane-row g holds
// r[j] = dword j of block g; on exit lane-row g holds in r[j] dword g of block j.
__device__ __forceinline__ void xpose4(const uint4& v, uint32_t* r) {
  const auto a = __builtin_amdgcn_permlane16_swap(v.x, v.y, false, false);
  const auto b = __builtin_amdgcn_permlane16_swap(v.z, v.w, false, false);
  const auto c = __builtin_amdgcn_permlane32_swap(a[0], b[0], false, false);
  const auto d = __builtin_amdgcn_permlane32_swap(a[1], b[1], false, false);
  r[0] = c[0];
  r[1] = d[0];
  r[2] = c[1];
  r[3] = d[1];
}

// How the remainder plane of the activation rows (XL::lo) enters a block:
//   LO_NONE  not at all (the rows are fp16-exact);
//   LO_STEP  a second product per step, into the same column.
constexpr int LO_NONE = 0, LO_STEP = 1;

// acc += one block for this lane's column: xh/xl point at the block's
// A operands of this lane (step t at +32 t elements), xs at its 4-sub-block
// sum group.  The row scale is applied by the caller.
template <int LOM>
__device__ __forceinline__ void q2_block(const uint4& qs, uint32_t scw, float d, float dmin,
                                         const _Float16* xh, const _Float16* xl,
                                         const _Float16* xs, f4_t& acc) {
  const f4_t zero = {0.f, 0.f, 0.f, 0.f};
  const uint32_t magic = q2_magic();
  const Q2Sc S = q2_scales(scw);
  f4_t dt = zero;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const h8_t b = q2_bop(qs, S, t, magic);
    dt = __builtin_amdgcn_mfma_f32_16x16x32_f16(*(const h8_t*)(xh + 32 * t), b, dt, 0, 0, 0);
    if (LOM == LO_STEP)
      dt = __builtin_amdgcn_mfma_f32_16x16x32_f16(*(const h8_t*)(xl + 32 * t), b, dt, 0, 0, 0);
  }
  const h8_t sx = *(const h8_t*)xs;
  const h4_t sxh = {sx[0], sx[1], sx[2], sx[3]}, sxl = {sx[4], sx[5], sx[6], sx[7]};
  // the 16-element sums are never fp16-exact: their remainder is always used
  f4_t dm = __builtin_amdgcn_mfma_f32_16x16x16f16(sxh, S.m, zero, 0, 0, 0);
  dm = __builtin_amdgcn_mfma_f32_16x16x16f16(sxl, S.m, dm, 0, 0, 0);
  const float nd = -dmin;
#pragma unroll
  for (int e = 0; e < 4; ++e) acc[e] = fmaf(nd, dm[e], fmaf(d, dt[e], acc[e]));
}

// fp16 value at position p (0..7) of an 8-value window held as 4 dwords.
__device__ __forceinline__ float win_val(const uint32_t* w, int p) {
  return f16bits_to_f32((uint16_t)(w[p >> 1] >> (16 * (p & 1))));
}

// Block scales d and dmin of blocks kb0..kb0+NBW-1 (fp32), from a chunk's loads.
template <int NBW, bool WIDE_D>
__device__ __forceinline__ void q2_chunk_scales(const Q2View& W, const Q2Chunk<NBW, WIDE_D>& c, int kb0, int n,
                                                float* dF, float* mF) {
  if (WIDE_D) {
    uint32_t dv[4], mv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w = j == 0 ? c.dd.x : j == 1 ? c.dd.y : j == 2 ? c.dd.z : c.dd.w;
      const auto s = __builtin_amdgcn_permlane16_swap(w, w, false, false);
      dv[j] = s[0];   // d of window blocks 2j, 2j + 1
      mv[j] = s[1];   // dmin of the same blocks
    }
    const int o = kb0 - q2_dwin(kb0, W.nb);   // wave-uniform offset of block kb0 in the window
    if (o <= 1) {
#pragma unroll
      for (int i = 0; i < NBW; ++i) {
        const int p1 = i + 1 < 8 ? i + 1 : 7;
        dF[i] = o ? win_val(dv, p1) : win_val(dv, i);
        mF[i] = o ? win_val(mv, p1) : win_val(mv, i);
      }
    } else {   // window clamped at the row end (shapes where a chunk starts late)
      const size_t rb = (size_t)n * W.nb + kb0;
#pragma unroll
      for (int i = 0; i < NBW; ++i) {
        dF[i] = f16bits_to_f32(W.d[rb + i]);
        mF[i] = f16bits_to_f32(W.dm[rb + i]);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < NBW; ++i) {
      dF[i] = f16bits_to_f32(c.d[WIDE_D ? 0 : i]);
      mF[i] = f16bits_to_f32(c.dm[WIDE_D ? 0 : i]);
    }
  }
}

// Blocks kb0..kb0+NBW-1 given their issued loads.
template <int NBW, bool WIDE_D, int LOM>
__device__ __forceinline__ void q2_chunk_compute(const Q2View& W, const Q2Chunk<NBW, WIDE_D>& c, int kb0,
                                        int n, const XL& X, int cr, int lane, f4_t& acc) {
  float dF[NBW], mF[NBW];
  q2_chunk_scales<NBW, WIDE_D>(W, c, kb0, n, dF, mF);
  const int g = lane >> 4;
  const _Float16* xh = X.hi + (size_t)cr * X.rs + kb0 * 256 + g * 8;
  const _Float16* xl = X.lo + (size_t)cr * X.rs + kb0 * 256 + g * 8;
  const _Float16* xs = X.sx + (size_t)cr * X.sxs + kb0 * 32 + g * 8;
  uint32_t sct[4];
#pragma unroll
  for (int i = 0; i < NBW; ++i) {
    if (i % 4 == 0) xpose4(c.sc[i / 4], sct);
    q2_block<LOM>(c.qs[i], sct[i % 4], dF[i], mF[i], xh + 256 * i, xl + 256 * i, xs + 32 * i,
                     acc);
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int NBW, bool WIDE_D, int LOM>
__device__ __forceinline__ void q2_chunk(const Q2View& W, int n, int kb0, const XL& X, int cr, int lane,
                                f4_t& acc) {
  Q2Chunk<NBW, WIDE_D> c;
  q2_chunk_load<NBW, WIDE_D>(W, n, kb0, lane >> 4, c);
  q2_chunk_compute<NBW, WIDE_D, LOM>(W, c, kb0, n, X, cr, lane, acc);
}

// Length of the chunk starting at kb with `left` blocks to go: at most WB,
// and 7 from an odd block so that its d/dmin window (even start) covers it.
template <bool WIDE_D>
__device__ __forceinline__ int q2_chunk_len(int kb, int left) {
  return min(left, (WIDE_D && (kb & 1)) ? WB - 1 : WB);
}

// Blocks [kb0, kb1) of row n, chunk by chunk.
template <bool WIDE_D, int LOM>
__device__ __forceinline__ void q2_range(const Q2View& W, int n, int kb0, int kb1, const XL& X, int cr,
                                int lane, f4_t& acc) {
  for (int kb = kb0; kb < kb1;) {
    const int len = q2_chunk_len<WIDE_D>(kb, kb1 - kb);
    switch (len) {
      case 1: q2_chunk<1, WIDE_D, LOM>(W, n, kb, X, cr, lane, acc); break;
      case 2: q2_chunk<2, WIDE_D, LOM>(W, n, kb, X, cr, lane, acc); break;
      case 3: q2_chunk<3, WIDE_D, LOM>(W, n, kb, X, cr, lane, acc); break;
      case 4: q2_chunk<4, WIDE_D, LOM>(W, n, kb, X, cr, lane, acc); break;
      case 5: q2_chunk<5, WIDE_D, LOM>(W, n, kb, X, cr, lane, acc); break;
      case 6: q2_chunk<6, WIDE_D, LOM>(W, n, kb, X, cr, lane, acc); break;
      case 7: q2_chunk<7, WIDE_D, LOM>(W, n, kb, X, cr, lane, acc); break;
      default: q2_chunk<8, WIDE_D, LOM>(W, n, kb, X, cr, lane, acc); break;
    }
    kb += len;
  }
}

// Number of vector loads q2_chunk_load issues for a chunk of NBW blocks when
// every load is 16 bytes wide (the compiler cannot merge those).  The narrow
// d/dmin loads may be merged into wider ones, so their count is unknown: 0
// then, and a wait for it waits for everything.
template <int NBW, bool WIDE_D>
constexpr int q2_chunk_nloads() {
  return WIDE_D ? NBW + (NBW + 3) / 4 + 1 : 0;
}

// Same as q2_range, for the start of a kernel: `issue()` runs first (it
// starts the loads that fill the LDS rows), then the first chunk's weight
// loads are issued, then `sync(n)` (n = the number of weight loads issued
// after issue()'s, so it can wait for exactly its own; it ends in a block
// barrier), then the blocks are computed.  Every wave calls both exactly once.
template <bool WIDE_D, int LOM, typename F, typename G>
__device__ __forceinline__ void q2_range_staged(const Q2View& W, int n, int kb0, int kb1,
                                                const XL& X, int cr, int lane, f4_t& acc,
                                                F&& issue, G&& sync) {
  const int len = q2_chunk_len<WIDE_D>(kb0, kb1 - kb0);
  const int g = lane >> 4;
  issue();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);   // the weight loads stay after issue()'s loads
#define SV_STAGED_CASE(L)                                               \
  case L: {                                                             \
    Q2Chunk<L, WIDE_D> c;                                               \
    q2_chunk_load<L, WIDE_D>(W, n, kb0, g, c);                          \
    sync(q2_chunk_nloads<L, WIDE_D>());                                 \
    q2_chunk_compute<L, WIDE_D, LOM>(W, c, kb0, n, X, cr, lane, acc);    \
    break;                                                              \
  }
  switch (len) {
    SV_STAGED_CASE(1)
    SV_STAGED_CASE(2)
    SV_STAGED_CASE(3)
    SV_STAGED_CASE(4)
    SV_STAGED_CASE(5)
    SV_STAGED_CASE(6)
    SV_STAGED_CASE(7)
    SV_STAGED_CASE(8)
    default: sync(0); return;   // empty range
  }
#undef SV_STAGED_CASE
  q2_range<WIDE_D, LOM>(W, n, kb0 + len, kb1, X, cr, lane, acc);
}

// Block barrier that does not wait for outstanding vector-memory loads (the
// compiler's __syncthreads() waits for all of them once LDS DMA is pending);
// compiler-only fences keep memory accesses on their side of it.  Callers make
// their own LDS writes complete first.  (Not inline asm: after an asm
// statement the compiler no longer knows which loads are outstanding and waits
// for all of them at the next use.)
__device__ __forceinline__ void barrier_keep_loads() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}


// Whether the 8-block d/dmin window loads apply to rows of nb blocks.
__host__ __device__ inline bool q2_wide_d(int nb) { return nb >= 8 && nb % 2 == 0; }

}  // namespace sv

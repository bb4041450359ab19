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

// bytes 0,1 (or 2,3) of u under the exponent byte of 1024.0: v_perm_b32 picks
// bytes 0-3 from its second operand and 4-7 from its first.
__device__ inline h2_t bytes01_to_h2(uint32_t u) {
  return __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u));
}
__device__ inline h2_t bytes23_to_h2(uint32_t u) {
  return __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u));
}

__device__ inline h8_t q8_bop(uint2 q) {
  const uint32_t a = q.x ^ 0x80808080u, b = q.y ^ 0x80808080u;
  const h2_t off = {(_Float16)1152.f, (_Float16)1152.f};
  const h2_t p0 = bytes01_to_h2(a) - off, p1 = bytes23_to_h2(a) - off;
  const h2_t p2 = bytes01_to_h2(b) - off, p3 = bytes23_to_h2(b) - off;
  h8_t r = {p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
  return r;
}

// One wave: T tiles of 16 vocabulary rows over all of K, in groups of 8 blocks
// (256 k, one activation-image scale per column).
//
// Loads: a lane reads 16 contiguous code bytes, so the 4 lanes of a row cover
// 64 bytes -- two blocks -- per instruction (32-byte pieces per row measure
// ~25% below the streaming read rate on this part; 64-byte pieces match it).
// One v_permlane32_swap per dword pair then gives every lane 8 bytes of each
// of the two blocks: lanes of k-group g hold block bytes 8*kofs(g)..+7 with
// kofs = (0, 2, 1, 3) for g = 0..3, and the activation operand is read at the
// same offsets.  Weight groups are double buffered: the loads of group j+1
// are issued before group j is computed.
template <int T, bool DVEC>
struct Q8Grp {
  uint4 q[T][4];     // 4 block pairs
  uint4 dv[T];
  uint16_t dd[T][DVEC ? 1 : 8];
};

template <int T, bool DVEC>
__device__ inline void q8_grp_load(const Q8View& W, const size_t* rowb, int kg, int nblk, int g,
                                   Q8Grp<T, DVEC>& G) {
#pragma unroll
  for (int t = 0; t < T; ++t) {
#pragma unroll
    for (int p = 0; p < 4; ++p)
      if (DVEC || 2 * p < nblk) G.q[t][p] = *(const uint4*)(W.qs + (rowb[t] + kg + 2 * p) * 32 + 16 * g);
    if (DVEC) {
      G.dv[t] = *(const uint4*)(W.d + rowb[t] + kg);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (i < nblk) G.dd[t][DVEC ? 0 : i] = W.d[rowb[t] + kg + i];
    }
  }
}

// Regroup one pair: returns (block A bytes, block B bytes) of this lane as uint2 each.
__device__ inline void q8_regroup(uint4 v, uint2& a, uint2& b) {
  const auto s0 = __builtin_amdgcn_permlane32_swap(v.x, v.z, false, false);
  const auto s1 = __builtin_amdgcn_permlane32_swap(v.y, v.w, false, false);
  a = make_uint2(s0[0], s1[0]);
  b = make_uint2(s0[1], s1[1]);
}

// DVEC: the block count is a multiple of 8, so every group is full -- no
// guards at all, and a group's 8 block scales come in one 16-byte load.
template <bool USE_LO, int T, bool DVEC>
__global__ __launch_bounds__(256) void k_q8_lmhead(Q8View W, int R, XImg img, float* logits) {
  const int lane = threadIdx.x & 63, wv = wave_id();
  const int tile0 = (blockIdx.x * 4 + wv) * T;
  const int vocab = W.n_out, K = W.nb * 32, nb = W.nb;
  if (tile0 * 16 >= vocab) return;
  const int nl = lane & 15, g = lane >> 4, cg = blockIdx.z;
  const int kofs = 8 * (((g & 1) << 1) | (g >> 1));   // k offset of this lane's 8 values in a block
  // padding columns read row R-1: an output column depends only on its own
  // operand row and padding columns are never stored, so every load stays
  // unconditional (branches around loads would serialise the memory waits)
  const int c = min(cg * 16 + nl, R - 1);
  const _Float16* xh = img.hi + (size_t)c * K + kofs;
  const _Float16* xl = img.lo + (size_t)c * K + kofs;
  size_t rowb[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int n = (tile0 + t) * 16 + nl;
    rowb[t] = (size_t)(n < vocab ? n : vocab - 1) * nb;   // ragged tail: valid row, result dropped
  }
  const f4_t zero = {0.f, 0.f, 0.f, 0.f};
  f4_t acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = zero;
  Q8Grp<T, DVEC> cur, nxt;
  q8_grp_load<T, DVEC>(W, rowb, 0, min(8, nb), g, cur);
  for (int kg = 0; kg < nb; kg += 8) {
    const int nblk = min(8, nb - kg);
    // issue order = use order: the loads retire in order, so the activation
    // operands of this group go out before the weights of the next one
    h8_t xa[8], xb[USE_LO ? 8 : 1];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (DVEC || i < nblk) {
        xa[i] = *(const h8_t*)(xh + (kg + i) * 32);
        if (USE_LO) xb[USE_LO ? i : 0] = *(const h8_t*)(xl + (kg + i) * 32);
      }
    }
    if (kg + 8 < nb) q8_grp_load<T, DVEC>(W, rowb, kg + 8, min(8, nb - kg - 8), g, nxt);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      if (DVEC || 2 * p < nblk) {
#pragma unroll
        for (int t = 0; t < T; ++t) {
          uint2 qa, qb;
          q8_regroup(cur.q[t][p], qa, qb);
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int i = 2 * p + h;
            if (DVEC || i < nblk) {
              const h8_t bw = q8_bop(h == 0 ? qa : qb);
              f4_t dt = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[i], bw, zero, 0, 0, 0);
              if (USE_LO) dt = __builtin_amdgcn_mfma_f32_16x16x32_f16(xb[USE_LO ? i : 0], bw, dt, 0, 0, 0);
              uint16_t db;
              if (DVEC) {
                const uint32_t w32 = p == 0 ? cur.dv[t].x : p == 1 ? cur.dv[t].y : p == 2 ? cur.dv[t].z : cur.dv[t].w;
                db = (uint16_t)(w32 >> (16 * h));
              } else {
                db = cur.dd[t][DVEC ? 0 : i];
              }
              const float d = f16b_to_f32(db);
#pragma unroll
              for (int e = 0; e < 4; ++e) acc[t][e] = fmaf(d, dt[e], acc[t][e]);
            }
          }
        }
      }
    }
    cur = nxt;
  }
  f4_t xs;   // row scales of the lane's 4 output columns
#pragma unroll
  for (int e = 0; e < 4; ++e) xs[e] = img.rscale[min(cg * 16 + 4 * g + e, R - 1)];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int n = (tile0 + t) * 16 + nl;
    if (n >= vocab) continue;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int cc = cg * 16 + 4 * g + e;
      if (cc < R) logits[(size_t)cc * vocab + n] = acc[t][e] * xs[e];
    }
  }
}

// ---------------------------------------------------------------------------
// Activation operands from LDS (block counts a multiple of 16).  Blocks of 8
// waves, 2 tiles per wave.  The block's columns are copied into LDS -- all of
// K at once when they fit (then there is no synchronisation in the K loop),
// else one window of `wg` groups at a time, double buffered, with one
// barrier per window (a window's copies are issued before the previous
// window is computed).  Every wave reads its activation operands from LDS
// instead of through the vector-memory path, which the weight stream then has
// to itself.
constexpr int LM_WAVES = 8, LM_T = 2;        // waves per block, tiles per wave
constexpr int LM_WIN_GROUPS = 4;             // window length (groups of 256 k) when K does not fit
constexpr size_t LM_LDS_CAP = 78 * 1024;     // two blocks per CU

struct LmCfg {
  int wg, nbuf, ncols, rs;   // window groups, buffers, columns per block, row stride (fp16)
  size_t lds;
};

static LmCfg lm_config(int K, int R, bool use_lo) {
  LmCfg c;
  c.ncols = R < 16 ? R : 16;
  const int ngroups = K / 256;
  const size_t pl = use_lo ? 2 : 1;
  c.wg = ngroups;
  c.nbuf = 1;
  c.rs = K + 8;
  if ((size_t)c.ncols * c.rs * 2 * pl > LM_LDS_CAP) {
    c.wg = LM_WIN_GROUPS;
    c.nbuf = 2;
    c.rs = LM_WIN_GROUPS * 256 + 8;
  }
  c.lds = (size_t)c.nbuf * c.ncols * c.rs * 2 * pl;
  return c;
}

// Copy window `wi` (wg groups) of columns c0 .. c0+nc-1 (hi, and lo when
// USE_LO) into buffer `buf`: 1 KB pieces, pieces w, w+8, ... to wave w.
template <bool USE_LO>
__device__ __forceinline__ void lm_window_dma(const XImg& img, int K, int c0, int nc, int wi, int buf,
                                              int wg, int nbuf, int ncols, int rs, uint32_t lds_base) {
  const int wv = wave_id(), lane = threadIdx.x & 63;
  const int ppc = wg * 256 * 2 / 1024;   // pieces per column and plane
  const int total = nc * ppc * (USE_LO ? 2 : 1);
  for (int q = wv; q < total; q += LM_WAVES) {
    const int pl = q / (nc * ppc), r = q - pl * nc * ppc, c = r / ppc, pc = r - c * ppc;
    const _Float16* src = (pl ? img.lo : img.hi) + (size_t)(c0 + c) * K + (size_t)wi * wg * 256 + pc * 512;
    const uint32_t la = lds_base + (uint32_t)((((pl * nbuf + buf) * ncols + c) * rs) * 2 + pc * 1024);
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"((const uint8_t*)src + 16 * lane), "s"(__builtin_amdgcn_readfirstlane(la))
                 : "memory", "m0");
  }
}

template <bool USE_LO>
__global__ __launch_bounds__(LM_WAVES * 64, 4) void k_q8_lmhead_lds(Q8View W, int R, XImg img, float* logits,
                                                                    LmCfg cfg) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int lane = threadIdx.x & 63, wv = wave_id();
  const int vocab = W.n_out, nb = W.nb, K = nb * 32;
  const int cg = blockIdx.z, c0 = cg * 16, nc = min(16, R - c0);
  const int wg = cfg.wg, nbuf = cfg.nbuf, ncols = cfg.ncols, rs = cfg.rs;
  const int tile0 = (blockIdx.x * LM_WAVES + wv) * LM_T;
  const int nl = lane & 15, g = lane >> 4;
  const int kofs = 8 * (((g & 1) << 1) | (g >> 1));   // k offset of this lane's 8 values in a block
  const uint32_t lds_base = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)lds;
  const _Float16* xw = (const _Float16*)lds;
  const int cr = min(nl, nc - 1);   // padding columns read the last real column; never stored
  size_t rowb[LM_T];
#pragma unroll
  for (int t = 0; t < LM_T; ++t) {
    const int n = (tile0 + t) * 16 + nl;
    // rows past the vocabulary (whole tiles past it included) read a valid row; dropped
    rowb[t] = (size_t)(n < vocab ? n : vocab - 1) * nb;
  }
  const int nwin = nb / (8 * wg);
  const f4_t zero = {0.f, 0.f, 0.f, 0.f};
  f4_t acc[LM_T];
#pragma unroll
  for (int t = 0; t < LM_T; ++t) acc[t] = zero;

  lm_window_dma<USE_LO>(img, K, c0, nc, 0, 0, wg, nbuf, ncols, rs, lds_base);
  Q8Grp<LM_T, true> ga, gb;
  q8_grp_load<LM_T, true>(W, rowb, 0, 8, g, ga);
  wait_vmcnt_le(5 * LM_T);   // window 0 copied (the group loads came after it)
  barrier_lds();
  for (int wi = 0; wi < nwin; ++wi) {
    const int buf = wi & 1;
    if (wi + 1 < nwin) lm_window_dma<USE_LO>(img, K, c0, nc, wi + 1, buf ^ 1, wg, nbuf, ncols, rs, lds_base);
    const _Float16* xh = xw + (size_t)(buf * ncols + cr) * rs + kofs;
    const _Float16* xl = xw + (size_t)((nbuf + buf) * ncols + cr) * rs + kofs;
    // one group: the next group's loads go out first, into the other buffer
    // (the two buffers alternate by name, so no copy waits on loads in flight)
    auto group = [&](int j, Q8Grp<LM_T, true>& cu, Q8Grp<LM_T, true>& nx) {
      const int kg = (wi * wg + j) * 8;
      // the last group's "next" loads re-read it (cache hits) so that every
      // path issues the same loads
      q8_grp_load<LM_T, true>(W, rowb, kg + 8 < nb ? kg + 8 : kg, 8, g, nx);
      __builtin_amdgcn_sched_barrier(0);   // keep them ahead of this group's math
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        // activation operands of blocks 2p, 2p+1 (read when needed: keeping a
        // group's worth live would not fit beside the double-buffered weights)
        h8_t xa[2], xb[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          xa[h] = *(const h8_t*)(xh + (j * 8 + 2 * p + h) * 32);
          if (USE_LO) xb[h] = *(const h8_t*)(xl + (j * 8 + 2 * p + h) * 32);
        }
#pragma unroll
        for (int t = 0; t < LM_T; ++t) {
          uint2 qa, qb;
          q8_regroup(cu.q[t][p], qa, qb);
          const uint32_t w32 = p == 0 ? cu.dv[t].x : p == 1 ? cu.dv[t].y : p == 2 ? cu.dv[t].z : cu.dv[t].w;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const h8_t bw = q8_bop(h == 0 ? qa : qb);
            f4_t dt = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[h], bw, zero, 0, 0, 0);
            if (USE_LO) dt = __builtin_amdgcn_mfma_f32_16x16x32_f16(xb[h], bw, dt, 0, 0, 0);
            const float d = f16b_to_f32((uint16_t)(w32 >> (16 * h)));
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[t][e] = fmaf(d, dt[e], acc[t][e]);
          }
        }
      }
    };
    // (wg is even; the buffers are back to (ga, gb) after every pair)
#pragma unroll 1
    for (int j = 0; j < wg; j += 2) {
      group(j, ga, gb);
      group(j + 1, gb, ga);
    }
    if (wi + 1 < nwin) {
      // this wave's copies of the next window were issued before the last
      // group's weight loads (5 per tile): wait for them, then for everyone
      wait_vmcnt_le(5 * LM_T);
      barrier_lds();
    }
  }
  f4_t xs;   // row scales of the lane's 4 output columns
#pragma unroll
  for (int e = 0; e < 4; ++e) xs[e] = img.rscale[min(c0 + 4 * g + e, R - 1)];
#pragma unroll
  for (int t = 0; t < LM_T; ++t) {
    const int n = (tile0 + t) * 16 + nl;
    if (n >= vocab) continue;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int cc = c0 + 4 * g + e;
      if (cc < R) logits[(size_t)cc * vocab + n] = acc[t][e] * xs[e];
    }
  }
}

// ---------------------------------------------------------------------------
// Weights streamed into LDS (block counts a multiple of 16, up to 8 columns;
// 4 with fp32 inputs; at most LD_MAX_ROUNDS tiles per wave).  Blocks of
// LD_WAVES (4 or 8) waves, persistent over tiles: in round r wave w of block
// b owns tile (r G + b) LD_WAVES + w.  Two 4-wave blocks per CU where both
// fit in LDS (each with its own stage barrier, so a slow wave holds up 3
// others, not 7), else one of 8 waves.  K is swept in stages of 16 blocks
// (512 k), stage-major: for each stage, the rounds' tiles one after another
// (one accumulator per round), so the block copies a stage's activation
// columns into its shared buffer once, not once per round.  For each step
// (stage, round) a wave copies its tile's 16 rows x 512 code bytes and
// 16 x 32 scale bytes into its own LDS buffer with global_load_lds (full
// 128-byte lines, non-temporal: this is the pattern that streams fastest on
// this part).  Everything is double buffered: step k+1 is in flight while
// step k is computed.  A wave waits only for its own copies before a step;
// the block meets once per stage, for the shared activation buffer.  Code
// rows are stored rotated by
// their row index in 16-byte units so that the 16 rows of an MFMA operand
// read fall in distinct LDS banks.
constexpr int LD_SB = 16;                                   // blocks (of 32) per stage
constexpr int LD_WBUF = 16 * LD_SB * 32;                    // code bytes per wave and stage (8 KB)
constexpr int LD_DBUF = 16 * LD_SB * 2;                     // scale bytes per wave and stage (512)
constexpr int LD_XRS = LD_SB * 32 + 8;                      // activation row stride (fp16)
constexpr int LD_XMAX = 8;                                  // columns (hi only; half with lo planes)
constexpr int LD_MAX_ROUNDS = 4;                            // tiles per wave (one accumulator each)

static size_t ld_lds_bytes(int waves, int ncols, bool use_lo) {
  return (size_t)waves * 2 * (LD_WBUF + LD_DBUF) + (size_t)2 * (use_lo ? 2 : 1) * ncols * LD_XRS * 2;
}
// SREG form: block scales in registers, activation rows unpadded (rotated)
static size_t ld_lds_bytes_sreg(int waves, int ncols, bool use_lo) {
  return (size_t)waves * 2 * LD_WBUF + (size_t)2 * (use_lo ? 2 : 1) * ncols * LD_SB * 32 * 2;
}


// Split over K (the products of small matrices, whose tiles alone would
// occupy few compute units): block (x, y, z) takes the stages [y sp, (y+1)
// sp) of matrix z (W, or W2 for z = 1) and writes its partial products to
// logits + z zstride + y R vocab (one [R, vocab] slice per y).  The head
// runs it with one slice (sp = all stages) and one matrix.
//
// SREG (8 waves, 16 columns): each lane loads its row's 16 block scales of a
// step into registers (two 16-byte loads, one step ahead, alternating
// between two register sets by round parity, so rounds come in pairs) instead
// of staging them in LDS, and an activation row of a stage is stored without
// padding, its 16-byte pieces rotated by the column index (piece p of column
// c at slot (p - c) mod 64) so that the 16 columns of an operand read still
// fall in distinct banks.  Then 8 waves' double-buffered weights and the
// activation buffers for 16 columns fit in the 160 KB of LDS, and the
// vocabulary takes 4 rounds of 8 waves per CU instead of 5 of 7.
template <bool USE_LO, int LD_WAVES, int MAXR = LD_MAX_ROUNDS, bool SREG = false>
__global__ __launch_bounds__(LD_WAVES * 64, 8 / LD_WAVES) void k_q8_lmhead_dma(Q8View W1, Q8View W2, int R,
                                                                               XImg img, float* logits,
                                                                               int ncols, int sp, size_t zstride) {
  static_assert(!SREG || MAXR % 2 == 0, "SREG rounds come in pairs");
  extern __shared__ __align__(16) uint8_t lds[];
  const Q8View W = blockIdx.z ? W2 : W1;
  const int lane = threadIdx.x & 63, wv = wave_id();
  const int vocab = W.n_out, nb = W.nb, K = nb * 32;
  const int tiles = (vocab + 15) / 16, st0 = blockIdx.y * sp, ns = min(st0 + sp, nb / LD_SB);
  logits += blockIdx.z * zstride + (size_t)blockIdx.y * R * vocab;
  // (SREG: always MAXR rounds, whose tiles past the last are skipped, so that
  // the scale registers take the same path through every stage)
  const int rounds = SREG ? MAXR : (tiles + gridDim.x * LD_WAVES - 1) / (gridDim.x * LD_WAVES);
  const int nl = lane & 15, g = lane >> 4;
  const int kofs = 8 * (((g & 1) << 1) | (g >> 1));   // k offset of this lane's 8 values in a block
  const uint32_t lbase = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)lds;
  constexpr int DBUF = SREG ? 0 : LD_DBUF;          // scale bytes per wave and stage in LDS
  constexpr int XRS = SREG ? LD_SB * 32 : LD_XRS;   // activation row stride (fp16)
  const uint32_t wbase = lbase + wv * 2 * LD_WBUF;
  const uint32_t dbase = lbase + LD_WAVES * 2 * LD_WBUF + wv * 2 * DBUF;
  const uint32_t xbase = lbase + LD_WAVES * 2 * (LD_WBUF + DBUF);
  const uint8_t* wl = lds + (wbase - lbase);
  const uint8_t* dl = lds + (dbase - lbase);
  const _Float16* xl16 = (const _Float16*)(lds + (xbase - lbase));
  const int cr = min(nl, ncols - 1);   // padding columns read the last real column; never stored
  const f4_t zero = {0.f, 0.f, 0.f, 0.f};

  // copies for step (stage st, round r) into weight buffer `wb` (wave-private
  // code and scale rows of the round's tile) and, for the first round of a
  // stage, the stage's activation columns into activation buffer `xb`
  // (shared by the block; column c by wave c mod LD_WAVES)
  // SREG: the scale registers of even and odd rounds
  uint4 sr[2][2];
  auto issue = [&](int st, int r, int wb, int xb, uint4 (&srn)[2]) {
    const int tile = (r * gridDim.x + blockIdx.x) * LD_WAVES + wv;
    if (SREG) {
      // this lane's row: its 16 block scales of the stage (loaded for every
      // tile, a row past the vocabulary reading the last one, so that the
      // registers are written on every path and are never copied while the
      // loads are in flight)
      const uint16_t* ds = W.d + (size_t)min(tile * 16 + nl, vocab - 1) * nb + st * LD_SB;
      srn[0] = *(const uint4*)ds;
      srn[1] = *(const uint4*)(ds + 8);
    }
    if (tile < tiles) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = 2 * i + (lane >> 5), c = lane & 31;
        const int n = min(tile * 16 + row, vocab - 1);
        const int8_t* src = W.qs + ((size_t)n * nb + st * LD_SB) * 32 + ((c + row) & 31) * 16;
        dma16_nt(src, wbase + wb * LD_WBUF + i * 1024);
      }
      if (!SREG && lane < 32) {   // scales: two 16-byte pieces per row, lanes 0..31
        const int row = lane >> 1;
        const int n = min(tile * 16 + row, vocab - 1);
        dma16(W.d + (size_t)n * nb + st * LD_SB + 8 * (lane & 1), dbase + wb * DBUF);
      }
    }
    if (r == 0)
      for (int c = wv; c < ncols * (USE_LO ? 2 : 1); c += LD_WAVES) {
        const int pl = c >= ncols, cc = c - (pl ? ncols : 0);
        const int piece = SREG ? ((lane + cc) & 63) : lane;
        const _Float16* src = (pl ? img.lo : img.hi) + (size_t)cc * K + st * LD_SB * 32 + 8 * piece;
        dma16(src, xbase + (uint32_t)(((pl * 2 + xb) * ncols + cc) * XRS * 2));
      }
  };

  // Stage-major: for each 512-k stage, every round's tile in turn, so a
  // stage's activation columns are copied once per block (not once per
  // round); each round keeps its own accumulator.
  f4_t acc[MAXR];
#pragma unroll
  for (int r = 0; r < MAXR; ++r) acc[r] = zero;
  issue(st0, 0, 0, st0 & 1, sr[0]);
  int k = 0;   // running step count: weight buffer k & 1
  for (int st = st0; st < ns; ++st) {
#pragma unroll
    for (int r = 0; r < MAXR; ++r) {
      if (r >= rounds) break;
      // this wave's copies of step k are done.  Weight buffers are private
      // to their wave, so only a stage's first step has a barrier: after it
      // every wave's activation copies of the stage are done, and every wave
      // is past stage st-1, whose activation buffer the copies of stage st+1
      // (issued in this stage's last round) reuse
      wait_vmcnt_le(0);
      if (r == 0) barrier_lds();
      if (r + 1 < rounds) issue(st, r + 1, (k + 1) & 1, st & 1, sr[(r + 1) & 1]);
      else if (st + 1 < ns) issue(st + 1, 0, (k + 1) & 1, (st + 1) & 1, sr[0]);
      const int tile = (r * gridDim.x + blockIdx.x) * LD_WAVES + wv;
      const int buf = k & 1, xbuf = st & 1;
      ++k;
      if (tile >= tiles) continue;
      const uint8_t* wb = wl + buf * LD_WBUF + nl * (LD_SB * 32);
      const _Float16* xh = xl16 + (size_t)(xbuf * ncols + cr) * XRS + (SREG ? 0 : kofs);
      const _Float16* xo = xl16 + (size_t)((2 + xbuf) * ncols + cr) * XRS + (SREG ? 0 : kofs);
      // activation operand of block blk: at blk * 32 + kofs, or (SREG) in the
      // rotated slot of that piece
      auto xat = [&](const _Float16* x, int blk) {
        return SREG ? *(const h8_t*)(x + 8 * ((4 * blk + (kofs >> 3) - cr) & 63))
                    : *(const h8_t*)(x + blk * 32);
      };
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        // 8 block scales of row nl
        const uint4 dv = SREG ? sr[r & 1][j] : *(const uint4*)(dl + buf * DBUF + nl * 32 + 16 * j);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int k16 = 16 * j + 4 * p + g;   // 16-byte piece of the row's stage bytes
          const uint4 qv = *(const uint4*)(wb + ((k16 - nl) & 31) * 16);
          uint2 qa, qb;
          q8_regroup(qv, qa, qb);
          const uint32_t w32 = p == 0 ? dv.x : p == 1 ? dv.y : p == 2 ? dv.z : dv.w;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int blk = j * 8 + 2 * p + h;
            const h8_t bw = q8_bop(h == 0 ? qa : qb);
            f4_t dt = __builtin_amdgcn_mfma_f32_16x16x32_f16(xat(xh, blk), bw, zero, 0, 0, 0);
            if (USE_LO) dt = __builtin_amdgcn_mfma_f32_16x16x32_f16(xat(xo, blk), bw, dt, 0, 0, 0);
            const float d = f16b_to_f32((uint16_t)(w32 >> (16 * h)));
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[r][e] = fmaf(d, dt[e], acc[r][e]);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);   // rounds one after another
    }
  }
#pragma unroll
  for (int r = 0; r < MAXR; ++r) {
    if (r >= rounds) break;
    const int tile = (r * gridDim.x + blockIdx.x) * LD_WAVES + wv;
    const int n = tile * 16 + nl;
    if (tile < tiles && n < vocab) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int cc = 4 * g + e;
        if (cc < R) logits[(size_t)cc * vocab + n] = acc[r][e] * img.rscale[cc];
      }
    }
  }
  wait_vmcnt_le(0);
}

// two tiles per wave: with double-buffered weight groups this keeps two waves
// per SIMD resident; 129280 rows then run in two full rounds of waves
template <bool USE_LO, int T>
static void launch_lm(int R, hipStream_t s, const Q8View& W, const XImg& img, float* logits) {
  const int tiles = (W.n_out + 15) / 16;
  const int waves = (tiles + T - 1) / T;
  const dim3 grid((waves + 3) / 4, 1, (R + 15) / 16);
  if (W.nb % 8 == 0)
    hipLaunchKernelGGL((k_q8_lmhead<USE_LO, T, true>), grid, dim3(256), 0, s, W, R, img, logits);
  else
    hipLaunchKernelGGL((k_q8_lmhead<USE_LO, T, false>), grid, dim3(256), 0, s, W, R, img, logits);
}

hipError_t launch_q8_lmhead(const void* w, int vocab, int hidden, int R, bool use_lo, XImg img,
                            float* logits, hipStream_t s) {
  const Q8View W = q8_view(w, vocab, hidden);
  const int ncu = cu_count();
  // two 4-wave blocks per CU when both fit in the CU's 160 KB of LDS
  const bool two = 2 * ld_lds_bytes(4, R, use_lo) <= (size_t)160 * 1024;
  const int waves = two ? 4 : 8;
  const long rounds = ((vocab + 15) / 16 + (long)(two ? 2 * ncu : ncu) * waves - 1) / ((long)(two ? 2 * ncu : ncu) * waves);
  if (W.nb % LD_SB == 0 && R <= (use_lo ? LD_XMAX / 2 : LD_XMAX) && rounds <= LD_MAX_ROUNDS) {
    const size_t lb = ld_lds_bytes(waves, R, use_lo);
    const dim3 grid(two ? 2 * ncu : ncu), block(waves * 64);
    const int ns = W.nb / LD_SB;
    if (use_lo) {
      if (two) hipLaunchKernelGGL((k_q8_lmhead_dma<true, 4>), grid, block, lb, s, W, W, R, img, logits, R, ns, (size_t)0);
      else hipLaunchKernelGGL((k_q8_lmhead_dma<true, 8>), grid, block, lb, s, W, W, R, img, logits, R, ns, (size_t)0);
    } else {
      if (two) hipLaunchKernelGGL((k_q8_lmhead_dma<false, 4>), grid, block, lb, s, W, W, R, img, logits, R, ns, (size_t)0);
      else hipLaunchKernelGGL((k_q8_lmhead_dma<false, 8>), grid, block, lb, s, W, W, R, img, logits, R, ns, (size_t)0);
    }
    return hipGetLastError();
  }
  // 9..16 rows (hi only; 5..8 with remainder planes): one block of eight
  // waves per CU with the scales in registers (the matrix-core tile has 16
  // columns, so the work per weight is that of 8 rows) while 4 rounds cover
  // the vocabulary, else seven waves, the activation buffer taking the LDS of
  // the eighth wave's weights, with up to eight tiles per wave
  {
    const long rounds8 = ((vocab + 15) / 16 + (long)ncu * 8 - 1) / ((long)ncu * 8);
    if (W.nb % LD_SB == 0 && R <= (use_lo ? LD_XMAX : 2 * LD_XMAX) && rounds8 <= LD_MAX_ROUNDS &&
        ld_lds_bytes_sreg(8, R, use_lo) <= (size_t)160 * 1024) {
      const size_t lb = ld_lds_bytes_sreg(8, R, use_lo);
      const int ns = W.nb / LD_SB;
      if (use_lo)
        hipLaunchKernelGGL((k_q8_lmhead_dma<true, 8, LD_MAX_ROUNDS, true>), dim3(ncu), dim3(8 * 64), lb, s, W, W, R,
                           img, logits, R, ns, (size_t)0);
      else
        hipLaunchKernelGGL((k_q8_lmhead_dma<false, 8, LD_MAX_ROUNDS, true>), dim3(ncu), dim3(8 * 64), lb, s, W, W,
                           R, img, logits, R, ns, (size_t)0);
      return hipGetLastError();
    }
  }
  {
    constexpr int W7 = 7;
    const long rounds7 = ((vocab + 15) / 16 + (long)ncu * W7 - 1) / ((long)ncu * W7);
    if (W.nb % LD_SB == 0 && R <= (use_lo ? LD_XMAX : 2 * LD_XMAX) && rounds7 <= 2 * LD_MAX_ROUNDS &&
        ld_lds_bytes(W7, R, use_lo) <= (size_t)160 * 1024) {
      const size_t lb = ld_lds_bytes(W7, R, use_lo);
      const int ns = W.nb / LD_SB;
      if (use_lo)
        hipLaunchKernelGGL((k_q8_lmhead_dma<true, W7, 2 * LD_MAX_ROUNDS>), dim3(ncu), dim3(W7 * 64), lb, s, W, W, R,
                           img, logits, R, ns, (size_t)0);
      else
        hipLaunchKernelGGL((k_q8_lmhead_dma<false, W7, 2 * LD_MAX_ROUNDS>), dim3(ncu), dim3(W7 * 64), lb, s, W, W, R,
                           img, logits, R, ns, (size_t)0);
      return hipGetLastError();
    }
  }
  // (groups in pairs; windows of LM_WIN_GROUPS groups when K does not fit)
  if (W.nb % (8 * LM_WIN_GROUPS) == 0) {
    const LmCfg cfg = lm_config(hidden, R, use_lo);
    const int tiles = (vocab + 15) / 16;
    const dim3 grid((tiles + LM_WAVES * LM_T - 1) / (LM_WAVES * LM_T), 1, (R + 15) / 16);
    if (use_lo)
      hipLaunchKernelGGL((k_q8_lmhead_lds<true>), grid, dim3(LM_WAVES * 64), cfg.lds, s, W, R, img, logits, cfg);
    else
      hipLaunchKernelGGL((k_q8_lmhead_lds<false>), grid, dim3(LM_WAVES * 64), cfg.lds, s, W, R, img, logits, cfg);
    return hipGetLastError();
  }
  if (use_lo)
    launch_lm<true, 2>(R, s, W, img, logits);
  else
    launch_lm<false, 2>(R, s, W, img, logits);
  return hipGetLastError();
}

int q8_split_parts(int vocab, int hidden, int R, bool use_lo, int nmat) {
  const int nb = hidden / 32, ns = nb / LD_SB, tiles = (vocab + 15) / 16;
  if (nb % LD_SB || R > LD_XMAX || ld_lds_bytes(4, R, use_lo) > (size_t)160 * 1024) return 0;
  // slices so that the launch has about two blocks per compute unit
  const int bx = (tiles + 3) / 4, want = 2 * cu_count();
  int sl = (want + bx * nmat - 1) / (bx * nmat);
  sl = sl < 1 ? 1 : (sl > ns ? ns : sl);
  const int sp = (ns + sl - 1) / sl;
  return (ns + sp - 1) / sp;
}

hipError_t launch_q8_split(const void* w1, const void* w2, int vocab, int hidden, int R, bool use_lo, XImg img,
                           float* part, hipStream_t s) {
  const int nmat = w2 ? 2 : 1, parts = q8_split_parts(vocab, hidden, R, use_lo, nmat);
  if (parts == 0) return hipErrorInvalidValue;
  const Q8View W1 = q8_view(w1, vocab, hidden), W2 = w2 ? q8_view(w2, vocab, hidden) : W1;
  const int ns = W1.nb / LD_SB, sp = (ns + parts - 1) / parts, tiles = (vocab + 15) / 16;
  const dim3 grid((tiles + 3) / 4, parts, nmat), block(256);
  const size_t lb = ld_lds_bytes(4, R, use_lo), zs = (size_t)parts * R * vocab;
  if (use_lo)
    hipLaunchKernelGGL((k_q8_lmhead_dma<true, 4>), grid, block, lb, s, W1, W2, R, img, part, R, sp, zs);
  else
    hipLaunchKernelGGL((k_q8_lmhead_dma<false, 4>), grid, block, lb, s, W1, W2, R, img, part, R, sp, zs);
  return hipGetLastError();
}

}  // namespace sv

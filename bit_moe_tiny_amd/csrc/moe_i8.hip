// The two-bit expert kernels of the MoE layer: gate/up + SwiGLU (k_gu8) and
// the down projection (k_dn8), on the int8 matrix cores with the weights
// streamed through LDS from the expert-tiled layout (sv_q2_tile in
// specverify.h: every step's codes, nibbles and scales are one contiguous
// chunk).
//
// Contraction (one 256-element block of 16 weight rows, one wave):
// v_mfma_i32_16x16x64_i8 with A = activation digits (tile column c = 4 slot
// + i: digit i of the descriptor's row `slot`), B = the weight
// bytes sc * q (at most 45), four products of 64 k per block (product t:
// sub-block 4g + t for lane group g); every product and every in-block sum is
// an exact integer.  The min term dmin * m * sum(x) is one 16x16x16 fp16
// product of the digit planes' sub-block sums (exact integers) with the m
// nibbles.  Block scales d, dmin are applied in fp32 per block; the digits are
// recombined (2^24, 2^16, 2^8, 1) and the row's power of two applied once at
// the end.  So the only roundings are the activations' (at most 2^-30 of
// their row's largest magnitude) and fp32 accumulation over the blocks.
//
// Weights are streamed ("Roofline" of the ds4-on-spark README: decode is
// bound by weight streaming): every wave keeps a ring of M8_RING slots, each
// holding one step -- one chunk of the tiled layout, two blocks (2688 bytes)
// or one (1344) of its 16 rows, read with three full-wave global-to-LDS
// instructions of 1 KB (non-temporal for pairs, whose chunks are whole
// 128-byte lines) -- and issues step j + M8_RING - 1 before computing step j.
// When a wave runs out of steps it issues placeholder loads of a chunk into a
// slot it never reads, so that every wait is the same constant vmcnt.  No block barrier is needed for
// weights: a wave only reads the slots its own loads filled.
//
// Work: persistent blocks of 8 waves, one per compute unit, each a contiguous
// range of items (all 8 waves on one item at a time):
//   k_gu8, MOE_ALLK descriptor (a unit of <= cap_allk rows): item = one
//     16-row tile of inter; wave (m, q): matrix m (gate, up), quarter q of
//     hidden.  The rows' digits over all of hidden stay in LDS.
//   k_gu8, MOE_QUARTER descriptor (a unit with more rows, e.g. the shared
//     expert): item = (quarter q, four 16-row tiles); wave (m, j): matrix m,
//     tile j of four, over quarter q; the rows' digits over that quarter stay
//     in LDS.
//   Either way every wave writes its quarter sums to the workspace; k_hdig
//     sums the quarters in order and applies SwiGLU.  Every weight tile is
//     read once.
//   k_dn8: item = eight 16-row tiles of hidden for one descriptor (at most
//     cap_down rows), wave j: tile j over all of inter.  The block copies the
//     descriptor's rows of the down input's digit image (written once per
//     assignment by k_hdig) into LDS when the descriptor changes.
// Blocks never wait on each other.
#include <type_traits>

#include "sv_digits.h"
#include "sv_internal.h"
#include "sv_q2.h"

namespace sv {

constexpr int M8_WAVES = 8, M8_THREADS = 64 * M8_WAVES;
constexpr int M8_RING = 4;                                   // steps per wave ring
constexpr int M8_CHUNK = 1344;                               // tiled bytes of one block of 16 rows
constexpr int M8_SLOT = 2 * M8_CHUNK;                        // one two-block step
constexpr int M8_DMA = 3;                                    // wave instructions per step
constexpr size_t M8_RINGS = (size_t)M8_WAVES * M8_RING * M8_SLOT;
constexpr size_t M8_RED = 64;                                // gate/up: row scales of the descriptor's columns
constexpr size_t M8_MISC = 256;                              // down: row maxima, flags, scales
constexpr size_t M8_LDS_MAX = 160 * 1024;
constexpr int M8_CAP_ALLK = 2;                               // rows of a MOE_ALLK descriptor, at most

// -------------------------------------------------------------- geometry
// LDS region of activation digits: ncols rows x 4 planes over nbr blocks,
// planes nbr*256 + 32 bytes apart, then the planes' sub-block sums (nbr*16
// fp16 each), nbr*32 + 16 bytes apart.  The paddings put the 16-byte (8-byte)
// pieces one operand read takes from different planes in different banks of
// the 64-bank LDS (measured: without them the reads take twice the cycles).
__host__ __device__ inline int m8_ps(int nbr) { return nbr * 256 + 32; }
__host__ __device__ inline int m8_ss(int nbr) { return nbr * 32 + 16; }
__host__ __device__ inline size_t m8_area(int nc, int nbr) {
  return (size_t)nc * NDIG * ((size_t)m8_ps(nbr) + (size_t)m8_ss(nbr));
}

static size_t gu_lds_bytes(int nc_allk, int nc_quarter, int nb) {
  const size_t a = m8_area(nc_allk, nb), q = m8_area(nc_quarter, (nb + 3) / 4);
  return M8_RINGS + M8_RED + (a > q ? a : q);
}
static size_t dn_lds_bytes(int nc, int nbd) { return M8_RINGS + M8_MISC + m8_area(nc, nbd); }

void moe8_caps(const sv_moe_desc* d, int* cap_allk, int* cap_quarter, int* cap_down) {
  const int nb = d->hidden / 256, nbd = d->inter / 256;
  int ca = M8_CAP_ALLK, cq = MOE_WORK_COLS, cd = MOE_WORK_COLS;
  while (ca > 1 && gu_lds_bytes(ca, 1, nb) > M8_LDS_MAX) --ca;
  while (cq > 1 && gu_lds_bytes(1, cq, nb) > M8_LDS_MAX) --cq;
  while (cd > 1 && dn_lds_bytes(cd, nbd) > M8_LDS_MAX) --cd;
  *cap_allk = ca;
  *cap_quarter = cq;
  *cap_down = cd;
}

bool moe_shape_ok(const sv_moe_desc* d) {
  if (d->hidden % 256 || d->inter % 256) return false;
  int ca, cq, cd;
  moe8_caps(d, &ca, &cq, &cd);
  return gu_lds_bytes(ca, cq, d->hidden / 256) <= M8_LDS_MAX &&
         dn_lds_bytes(cd, d->inter / 256) <= M8_LDS_MAX;
}

// ----------------------------------------------------------------- steps
// Blocks [b0, b1) of a row as steps (the grouping of the tiled layout): a step
// at an odd block, or at the last block, holds one block; every other step an
// aligned pair.

__device__ __forceinline__ bool m8_pair(int kb, int b1) { return !(kb & 1) && kb + 1 < b1; }

// The M8_DMA wave instructions of one step: the chunk at p (1344 bytes per
// block) into the slot at LDS byte address sa, every lane copying 16 bytes
// at offset 16 lane of each 1 KB piece.  A pair (2688 bytes, whole 128-byte
// lines, non-temporal) is read as the pieces at 0, 1024 and 1664, a single
// block (1344 bytes) as the pieces at 0, 160 and 320: the last piece
// overlaps the one before it inside the chunk (those bytes land twice, with
// the same values), so every lane of every instruction copies bytes of the
// chunk into the chunk's place in the slot, with no lane masked.
__device__ __forceinline__ void m8_issue(const uint8_t* p, bool pair, uint32_t voff, uint32_t sa) {
  if (pair) {
    dma16s_nt(p, voff, sa);
    dma16s_nt(p + 1024, voff, sa + 1024);
    dma16s_nt(p + 1664, voff, sa + 1664);
  } else {
    dma16s(p, voff, sa);
    dma16s(p + 160, voff, sa + 160);
    dma16s(p + 320, voff, sa + 320);
  }
}

// Placeholder for a step past the end of the wave's work: the M8_DMA loads
// of a single-block step from p (any chunk's first 1344 bytes) into the slot
// at sa, which is never read.
__device__ __forceinline__ void m8_issue_none(const uint8_t* p, uint32_t voff, uint32_t sa) {
  dma16s(p, voff, sa);
  dma16s(p + 160, voff, sa + 160);
  dma16s(p + 320, voff, sa + 320);
}

// The wait before computing a step: the oldest of M8_RING steps in flight is
// complete (vector-memory loads complete in order; outstanding stores only
// make the wait longer).
__device__ __forceinline__ void m8_wait_step() { wait_vmcnt_le(M8_DMA * (M8_RING - 1)); }

// ------------------------------------------------------------ contraction
// Lane (n, g) pointers into the digit region for column tile ct: the lane's
// tile column c = lane & 15 is digit c & 3 of row slot min(4 ct + c / 4,
// nc - 1) (columns past the rows repeat the last row; their results are
// never stored).
struct M8A {
  const int8_t* a[2];
  const _Float16* s[2];
};

__device__ __forceinline__ M8A m8_aptr(const uint8_t* reg, int nc, int nbr, int lane) {
  M8A p;
  const int c = lane & 15, g = lane >> 4;
  const _Float16* sx = (const _Float16*)(reg + (size_t)nc * NDIG * m8_ps(nbr));
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int slot = min(4 * ct + (c >> 2), nc - 1), pl = slot * NDIG + (c & 3);
    p.a[ct] = (const int8_t*)(reg + (size_t)pl * m8_ps(nbr) + 16 * g);
    p.s[ct] = sx + (size_t)pl * (m8_ss(nbr) / 2) + 4 * g;
  }
  return p;
}

typedef int i4_t __attribute__((ext_vector_type(4)));

typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

// Weight bytes sc * q of one sub-block dword w as the four B-operand dwords of
// its product (sc2: sc in both 16-bit halves): byte b of dword j is code
// 4b + j.  One packed 16-bit multiply per dword: each 16-bit half holds two
// codes (bytes), and (256 q1 + q0) sc stays below 2^16 (sc q <= 45), so the
// bytes stay apart.
__device__ __forceinline__ i4_t m8_bop(uint32_t w, uint32_t sc2) {
  const uint32_t m = 0x03030303u;
  const u16x2_t s2 = __builtin_bit_cast(u16x2_t, sc2);
  i4_t b;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    b[j] = (int)__builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2_t, (w >> (2 * j)) & m) * s2);
  return b;
}

// acc[ct] += one step of NB blocks (the chunk in slot; kbl = the first
// block's index in the digit region) for column tiles ct < NCT.  Every LDS
// read of the step is issued first -- weights, scales, activation digits and
// their sums of both blocks -- so that the wave waits once, then the blocks'
// matrix products are interleaved (independent accumulators).  Slot offsets
// follow the chunk layout: codes of row n, piece c at 64 NB n + 16 ((c + n)
// mod 4 NB); the nibble dword g of block b, row n at 1024 NB + 4 (16 (4 b +
// g) + n); d, dmin at 1280 NB and 1312 NB, NB halves per row.
template <int NB, int NCT>
__device__ __forceinline__ void m8_step_compute(const uint8_t* slot, int kbl, const M8A& A, f4_t (&acc)[2]) {
  const int lane = __lane_id(), n = lane & 15, g = lane >> 4;
  uint4 qs[NB];
  uint32_t scw[NB];
  i4_t xa[NB][NCT][4];
  h4_t sx[NB][NCT];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    qs[b] = *(const uint4*)(slot + n * 64 * NB + (((4 * b + g + n) & (4 * NB - 1)) << 4));
    scw[b] = *(const uint32_t*)(slot + 1024 * NB + ((b * 4 + g) * 16 + n) * 4);
  }
  uint32_t dw, mw;
  if (NB == 2) {
    dw = *(const uint32_t*)(slot + 2560 + n * 4);
    mw = *(const uint32_t*)(slot + 2624 + n * 4);
  } else {
    dw = *(const uint16_t*)(slot + 1280 + n * 2);
    mw = *(const uint16_t*)(slot + 1312 + n * 2);
  }
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int8_t* xp = A.a[ct] + (size_t)(kbl + b) * 256;
#pragma unroll
      for (int t = 0; t < 4; ++t) xa[b][ct][t] = *(const i4_t*)(xp + 64 * t);
      sx[b][ct] = *(const h4_t*)(A.s[ct] + (size_t)(kbl + b) * 16);
    }
  const h2_t k1024 = {(_Float16)1024.f, (_Float16)1024.f};
  const f4_t zero = {0.f, 0.f, 0.f, 0.f};
  i4_t B[NB][4];
  h4_t m[NB];
  float d[NB], dmin[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const uint32_t sc4 = scw[b] & 0x0F0F0F0Fu;
#pragma unroll
    for (int t = 0; t < 4; ++t)
      B[b][t] = m8_bop(t == 0 ? qs[b].x : t == 1 ? qs[b].y : t == 2 ? qs[b].z : qs[b].w,
                       __builtin_amdgcn_perm(0u, sc4, 0x0C000C00u | (uint32_t)(t * 0x00010001)));
    const uint32_t mh = (scw[b] >> 4) & 0x0F0F0F0Fu;
    const h2_t m01 = q2_bytes01(mh) - k1024, m23 = q2_bytes23(mh) - k1024;
    m[b] = (h4_t){m01.x, m01.y, m23.x, m23.y};
    d[b] = f16bits_to_f32((uint16_t)(dw >> (16 * b)));
    dmin[b] = f16bits_to_f32((uint16_t)(mw >> (16 * b)));
  }
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    i4_t D[NB];
    f4_t dm[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) D[b] = (i4_t){0, 0, 0, 0};
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int b = 0; b < NB; ++b) D[b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(xa[b][ct][t], B[b][t], D[b], 0, 0, 0);
#pragma unroll
    for (int b = 0; b < NB; ++b) dm[b] = __builtin_amdgcn_mfma_f32_16x16x16f16(sx[b][ct], m[b], zero, 0, 0, 0);
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[ct][e] = fmaf(-dmin[b], dm[b][e], fmaf(d[b], (float)D[b][e], acc[ct][e]));
  }
}


// The same loads with one M0 and one base for all pieces of a step: the
// instruction offset moves the global and the LDS address alike.
__device__ __forceinline__ void m8_issue_o(const uint8_t* p, bool pair, uint32_t voff, uint32_t sa) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(sa);
  if (pair)
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "global_load_lds_dwordx4 %0, %1 nt\n\t"
        "global_load_lds_dwordx4 %0, %1 offset:1024 nt\n\t"
        "global_load_lds_dwordx4 %0, %1 offset:1664 nt"
        :: "v"(voff), "s"(p), "s"(m0) : "memory", "m0");
  else
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "global_load_lds_dwordx4 %0, %1\n\t"
        "global_load_lds_dwordx4 %0, %1 offset:160\n\t"
        "global_load_lds_dwordx4 %0, %1 offset:320"
        :: "v"(voff), "s"(p), "s"(m0) : "memory", "m0");
}

// Step patterns of the items whose block range is four steps long (the
// grouping of the tiled layout): blocks per step, the step's first block
// relative to the item's, and its chunk offset.
template <int N0, int N1, int N2, int N3>
struct M8Pat {
  static constexpr int nb(int j) { return j == 0 ? N0 : j == 1 ? N1 : j == 2 ? N2 : N3; }
  static constexpr int rel(int j) { return j == 0 ? 0 : rel(j - 1) + nb(j - 1); }
  static constexpr int off(int j) { return M8_CHUNK * rel(j); }
};
using M8PatA = M8Pat<2, 2, 2, 1>;   // 7 blocks from an even block
using M8PatB = M8Pat<1, 2, 2, 2>;   // 7 blocks from an odd block
using M8PatC = M8Pat<2, 2, 2, 2>;   // 8 blocks from an even block

// One step of an unrolled item: wait for its loads, contract, release the slot.
template <class PAT, int NCT, int J>
__device__ __forceinline__ void m8_fstep(const uint8_t* ring, const M8A& A, f4_t (&acc)[2]) {
  m8_wait_step();
  m8_step_compute<PAT::nb(J), NCT>(ring + J * M8_SLOT, PAT::rel(J), A, acc);
  __builtin_amdgcn_s_waitcnt(0xC07F);   // this slot's LDS reads are done before it is refilled
}

// The four steps of an item in slots 0..3; after step j, nx(j) issues step j
// of the next item into the freed slot j, so the loads of the rest of this
// item and the start of the next (three steps) are in flight during every
// contraction and each wait is the same count.
template <class PAT, int NCT, class NX>
__device__ __forceinline__ void m8_fitem(const uint8_t* ring, const M8A& A, f4_t (&acc)[2], NX& nx) {
  m8_fstep<PAT, NCT, 0>(ring, A, acc);
  nx(std::integral_constant<int, 0>());
  m8_fstep<PAT, NCT, 1>(ring, A, acc);
  nx(std::integral_constant<int, 1>());
  m8_fstep<PAT, NCT, 2>(ring, A, acc);
  nx(std::integral_constant<int, 2>());
  m8_fstep<PAT, NCT, 3>(ring, A, acc);
  nx(std::integral_constant<int, 3>());
}

// The digits of a row slot recombined (fixed order).
__device__ __forceinline__ float m8_value(const f4_t& a) {
  return fmaf(a[0], 16777216.f, a[1] * 65536.f) + fmaf(a[2], 256.f, a[3]);
}


// Copies n bytes (a multiple of 16) from global memory into LDS at byte
// address la, 1 KB per wave instruction, pieces distributed over the block's
// waves starting at piece index *q.
__device__ __forceinline__ void m8_copy(const void* src, uint32_t la, int n, int& q) {
  const int lane = threadIdx.x & 63, wv = wave_id();
  for (int o = 0; o < n; o += 1024, ++q) {
    if ((q & (M8_WAVES - 1)) != wv) continue;
    if (o + 16 * lane < n) dma16((const uint8_t*)src + o + 16 * lane, la + o);
  }
}

// Rows rows[0..nc) of the digit image over blocks [rb0, rb0 + nbr) into the
// region at reg (whole block; completion is the caller's wait).
__device__ void m8_load_x(const XDig& xd, const int* rows, int nc, int rb0, int nbr, uint8_t* reg) {
  const int K = xd.K;
  const uint32_t la = lds_addr(reg);
  const uint32_t las = la + (uint32_t)((size_t)nc * NDIG * m8_ps(nbr));
  int q = 0;
  for (int c = 0; c < nc; ++c) {
    const int r = rows[c];
    for (int i = 0; i < NDIG; ++i) {
      const int pl = c * NDIG + i;
      m8_copy(xd.dig + ((size_t)r * NDIG + i) * K + (size_t)rb0 * 256, la + (uint32_t)pl * m8_ps(nbr), nbr * 256, q);
      m8_copy(xd.sx + ((size_t)r * NDIG + i) * (K / 16) + (size_t)rb0 * 16, las + (uint32_t)pl * m8_ss(nbr), nbr * 32, q);
    }
  }
}

// ----------------------------------------------------------------- gate/up
struct ExpertPtrs {
  const uint8_t *g, *u, *dn;     // routed, expert-major, tiled
  const uint8_t *sg, *su, *sd;   // shared
  size_t bytes_gu, bytes_d;
};

static ExpertPtrs expert_ptrs(const sv_moe_desc* d) {
  ExpertPtrs P;
  P.g = (const uint8_t*)d->w_gate;
  P.u = (const uint8_t*)d->w_up;
  P.dn = (const uint8_t*)d->w_down;
  P.sg = (const uint8_t*)d->s_gate;
  P.su = (const uint8_t*)d->s_up;
  P.sd = (const uint8_t*)d->s_down;
  P.bytes_gu = q2_tiled_bytes(d->inter, d->hidden);
  P.bytes_d = q2_tiled_bytes(d->hidden, d->inter);
  return P;
}

// Position in a block's item range: descriptor d, item l of its T, and for
// MOE_QUARTER descriptors the quarter q and tile group gq (l = q T/4 + gq),
// advanced one item at a time (no divisions in the loop).
struct GuCur {
  int d, l, q, gq, type, e;
};

// The work of one wave on an item: its tile over blocks [b0, b1) (a quarter),
// whose first chunk is at p.
struct GuItem {
  int tile, q, b0, b1;
  const uint8_t* p;
};

// Runs the steps of one item (template on the column tiles), issuing the
// load cursor's next step before each.
template <int NCT, typename Issue>
__device__ __forceinline__ void m8_item(const uint8_t* ring, int& cslot, int b0, int b1, int rb0, const M8A& A,
                                        f4_t (&acc)[2], Issue& issue) {
  for (int kb = b0; kb < b1;) {
    issue();
    m8_wait_step();
    const uint8_t* slot = ring + cslot * M8_SLOT;
    if (m8_pair(kb, b1)) {
      m8_step_compute<2, NCT>(slot, kb - rb0, A, acc);
      kb += 2;
    } else {
      m8_step_compute<1, NCT>(slot, kb - rb0, A, acc);
      kb += 1;
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);   // this slot's LDS reads are done before it is refilled
    cslot = cslot == M8_RING - 1 ? 0 : cslot + 1;
  }
}

__global__ __launch_bounds__(M8_THREADS, 1) void k_gu8(ExpertPtrs P, int nb, int inter, MoeWs ws) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int T = inter / 16, G4 = T / 4;
  const auto work = const_ptr(ws.work_gu);
  const int nd = const_ptr(ws.meta)->n_work_gu;
  const int i0 = const_ptr(ws.blk_gu)[blockIdx.x], i1 = const_ptr(ws.blk_gu)[blockIdx.x + 1];
  if (i0 >= i1) return;
  const int lane = threadIdx.x & 63, w = wave_id();
  const int mm = w >> 2, wj = w & 3;
  const int n = lane & 15, g = lane >> 4;
  uint8_t* ring = lds + (size_t)w * M8_RING * M8_SLOT;
  const uint32_t ring_la = lds_addr(ring);
  float* s_rsc = (float*)(lds + M8_RINGS);   // row scales of the current descriptor's columns
  uint8_t* reg = lds + M8_RINGS + M8_RED;
  const uint32_t voff = 16u * (uint32_t)lane;
  const uint8_t* const mroute = mm == 0 ? P.g : P.u;
  const uint8_t* const mshared = mm == 0 ? P.sg : P.su;

  auto cur_at = [&](int i) {
    GuCur c;
    c.d = i / T;
    c.l = i - c.d * T;
    c.q = c.l / G4;
    c.gq = c.l - c.q * G4;
    c.type = work[c.d].type;
    c.e = work[c.d].expert;
    return c;
  };
  auto advance = [&](GuCur& c) {
    if (++c.l == T) {
      if (++c.d < nd) {
        c.type = work[c.d].type;
        c.e = work[c.d].expert;
      }
      c.l = c.q = c.gq = 0;
    } else if (++c.gq == G4) {
      c.gq = 0;
      ++c.q;
    }
  };
  auto item = [&](const GuCur& c) {
    GuItem u;
    if (c.type == MOE_ALLK) {
      u.tile = c.l;
      u.q = wj;
    } else {
      u.tile = c.gq * 4 + wj;
      u.q = c.q;
    }
    u.b0 = (nb * u.q) >> 2;
    u.b1 = (nb * (u.q + 1)) >> 2;
    const uint8_t* mat = c.e >= 0 ? mroute + (size_t)c.e * P.bytes_gu : mshared;
    u.p = mat + (size_t)M8_CHUNK * ((size_t)u.tile * nb + u.b0);
    return u;
  };

  // load cursor: the step at block lkb of item lu (chunk lp; lleft items
  // left, counting this one), into ring slot lslot
  GuCur lc = cur_at(i0);
  GuItem lu = item(lc);
  int lleft = i1 - i0, lkb = lu.b0, lslot = 0;
  const uint8_t* lp = lu.p;
  const uint8_t* const pvalid = lu.p;   // a readable address for placeholder loads
  auto skip = [&]() {
    while (lleft > 0 && lkb >= lu.b1) {
      if (--lleft > 0) {
        advance(lc);
        lu = item(lc);
        lkb = lu.b0;
        lp = lu.p;
      }
    }
  };
  skip();
  auto issue = [&]() {
    const uint32_t sa = ring_la + (uint32_t)(lslot * M8_SLOT);
    if (lleft > 0) {
      const bool pair = m8_pair(lkb, lu.b1);
      m8_issue(lp, pair, voff, sa);
      lkb += pair ? 2 : 1;
      lp += pair ? M8_SLOT : M8_CHUNK;
      skip();
    } else {
      m8_issue_none(pvalid, voff, sa);
    }
    lslot = lslot == M8_RING - 1 ? 0 : lslot + 1;
  };
  for (int k = 0; k < M8_RING - 1; ++k) issue();

  GuCur cc = cur_at(i0);
  int cslot = 0, key_d = -1, key_q = -2, nc = 1, a0 = 0, rb0 = 0;
  M8A A = m8_aptr(reg, 1, 1, lane);
  for (int it = i0; it < i1; ++it, advance(cc)) {
    const GuItem cu = item(cc);
    const int kq = cc.type == MOE_ALLK ? -1 : cu.q;
    if (cc.d != key_d || kq != key_q) {
      // a new set of activation rows: every wave is past the old ones
      barrier_lds();
      nc = work[cc.d].ncols;
      a0 = work[cc.d].a0;
      rb0 = cc.type == MOE_ALLK ? 0 : cu.b0;
      const int nbr = cc.type == MOE_ALLK ? nb : cu.b1 - cu.b0;
      int rows[MOE_WORK_COLS];
#pragma unroll
      for (int c = 0; c < MOE_WORK_COLS; ++c) rows[c] = work[cc.d].rows[c];
      m8_load_x(ws.xd, rows, nc, rb0, nbr, reg);
      if (threadIdx.x < MOE_WORK_COLS) s_rsc[threadIdx.x] = ws.xd.rsc[rows[min((int)threadIdx.x, nc - 1)]];
      wait_vmcnt_le(0);
      barrier_lds();
      key_d = cc.d;
      key_q = kq;
      A = m8_aptr(reg, nc, nbr, lane);
    }
    f4_t acc[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) acc[ct] = (f4_t){0.f, 0.f, 0.f, 0.f};
    if (nc <= 4) m8_item<1>(ring, cslot, cu.b0, cu.b1, rb0, A, acc, issue);
    else m8_item<2>(ring, cslot, cu.b0, cu.b1, rb0, A, acc, issue);
    {
      // this wave's quarter sums of its tile, per row slot, to the workspace
      // (k_hdig sums the quarters and applies SwiGLU)
      const int nct = (nc + 3) / 4;
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const int sl = 4 * ct + g;
        if (ct < nct && sl < nc) {
          const float rs = s_rsc[sl];
          ws.gpart[(((size_t)mm * 4 + cu.q) * ws.max_assign + a0 + sl) * inter + cu.tile * 16 + n] =
              m8_value(acc[ct]) * rs;
        }
      }
    }
  }
  wait_vmcnt_le(0);
}

// The same work for a hidden size of 4*NQ blocks with NQ = 7 or 8, where
// every wave's part of an item is exactly four steps (patterns A/B for a
// quarter of 7 blocks starting at an even/odd block, C for 8): the item body
// is unrolled with the ring slots, step offsets and digit offsets fixed at
// compile time, and the loads run one item ahead (m8_fitem).
template <int NQ>
__global__ __launch_bounds__(M8_THREADS, 1) void k_gu8f(ExpertPtrs P, int inter, MoeWs ws) {
  using PE = typename std::conditional<NQ == 7, M8PatA, M8PatC>::type;   // quarters from an even block
  using PO = M8PatB;                                                      // (NQ = 7) from an odd block
  constexpr int nb = 4 * NQ;
  extern __shared__ __align__(16) uint8_t lds[];
  const int T = inter / 16, G4 = T / 4;
  const auto work = const_ptr(ws.work_gu);
  const int nd = const_ptr(ws.meta)->n_work_gu;
  const int i0 = const_ptr(ws.blk_gu)[blockIdx.x], i1 = const_ptr(ws.blk_gu)[blockIdx.x + 1];
  if (i0 >= i1) return;
  const int lane = threadIdx.x & 63, w = wave_id();
  const int mm = w >> 2, wj = w & 3;
  const int n = lane & 15, g = lane >> 4;
  uint8_t* ring = lds + (size_t)w * M8_RING * M8_SLOT;
  const uint32_t ring_la = lds_addr(ring);
  float* s_rsc = (float*)(lds + M8_RINGS);   // row scales of the current descriptor's columns
  uint8_t* reg = lds + M8_RINGS + M8_RED;
  const uint32_t voff = 16u * (uint32_t)lane;
  const uint8_t* const mroute = mm == 0 ? P.g : P.u;
  const uint8_t* const mshared = mm == 0 ? P.sg : P.su;

  auto cur_at = [&](int i) {
    GuCur c;
    c.d = i / T;
    c.l = i - c.d * T;
    c.q = c.l / G4;
    c.gq = c.l - c.q * G4;
    c.type = work[c.d].type;
    c.e = work[c.d].expert;
    return c;
  };
  auto advance = [&](GuCur& c) {
    if (++c.l == T) {
      if (++c.d < nd) {
        c.type = work[c.d].type;
        c.e = work[c.d].expert;
      }
      c.l = c.q = c.gq = 0;
    } else if (++c.gq == G4) {
      c.gq = 0;
      ++c.q;
    }
  };
  auto item = [&](const GuCur& c) {
    GuItem u;
    if (c.type == MOE_ALLK) {
      u.tile = c.l;
      u.q = wj;
    } else {
      u.tile = c.gq * 4 + wj;
      u.q = c.q;
    }
    u.b0 = NQ * u.q;
    u.b1 = u.b0 + NQ;
    const uint8_t* mat = c.e >= 0 ? mroute + (size_t)c.e * P.bytes_gu : mshared;
    u.p = mat + (size_t)M8_CHUNK * ((size_t)u.tile * nb + u.b0);
    return u;
  };

  // step j of the item at p (odd: its quarter starts at an odd block) into
  // slot j; p == nullptr: a placeholder
  auto issue = [&](auto J, const uint8_t* p, bool odd) {
    constexpr int j = decltype(J)::value;
    const uint32_t sa = ring_la + (uint32_t)(j * M8_SLOT);
    if (p == nullptr) {
      m8_issue_none(P.sg ? P.sg : P.g, voff, sa);
      return;
    }
    const int off = odd ? PO::off(j) : PE::off(j);
    const bool pair = odd ? PO::nb(j) == 2 : PE::nb(j) == 2;
    m8_issue_o(p + off, pair, voff, sa);
  };

  GuCur cc = cur_at(i0);
  GuItem cu = item(cc);
  {
    const bool odd = cu.b0 & 1;
    issue(std::integral_constant<int, 0>(), cu.p, odd);
    issue(std::integral_constant<int, 1>(), cu.p, odd);
    issue(std::integral_constant<int, 2>(), cu.p, odd);
    issue(std::integral_constant<int, 3>(), cu.p, odd);
  }
  int key_d = -1, key_q = -2, nc = 1, a0 = 0;
  M8A A = m8_aptr(reg, 1, 1, lane);
  for (int it = i0; it < i1; ++it) {
    // the next item, whose loads start during this one
    GuCur nc_ = cc;
    const uint8_t* np = nullptr;
    bool nodd = false;
    if (it + 1 < i1) {
      advance(nc_);
      const GuItem nu = item(nc_);
      np = nu.p;
      nodd = nu.b0 & 1;
    }
    const int kq = cc.type == MOE_ALLK ? -1 : cu.q;
    if (cc.d != key_d || kq != key_q) {
      // a new set of activation rows: every wave is past the old ones
      barrier_lds();
      nc = work[cc.d].ncols;
      a0 = work[cc.d].a0;
      const int rb0 = cc.type == MOE_ALLK ? 0 : cu.b0;
      const int nbr = cc.type == MOE_ALLK ? nb : NQ;
      int rows[MOE_WORK_COLS];
#pragma unroll
      for (int c = 0; c < MOE_WORK_COLS; ++c) rows[c] = work[cc.d].rows[c];
      m8_load_x(ws.xd, rows, nc, rb0, nbr, reg);
      if (threadIdx.x < MOE_WORK_COLS) s_rsc[threadIdx.x] = ws.xd.rsc[rows[min((int)threadIdx.x, nc - 1)]];
      wait_vmcnt_le(0);
      barrier_lds();
      key_d = cc.d;
      key_q = kq;
      A = m8_aptr(reg, nc, nbr, lane);
      if (cc.type == MOE_ALLK) {   // this wave's quarter of the rows
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          A.a[ct] += (size_t)cu.b0 * 256;
          A.s[ct] += (size_t)cu.b0 * 16;
        }
      }
    }
    f4_t acc[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) acc[ct] = (f4_t){0.f, 0.f, 0.f, 0.f};
    auto nx = [&](auto J) { issue(J, np, nodd); };
    const bool odd = cu.b0 & 1;
    if (nc <= 4) {
      if (NQ == 7 && odd) m8_fitem<PO, 1>(ring, A, acc, nx);
      else m8_fitem<PE, 1>(ring, A, acc, nx);
    } else {
      if (NQ == 7 && odd) m8_fitem<PO, 2>(ring, A, acc, nx);
      else m8_fitem<PE, 2>(ring, A, acc, nx);
    }
    {
      // this wave's quarter sums of its tile, per row slot, to the workspace
      // (k_hdig sums the quarters and applies SwiGLU)
      const int nct = (nc + 3) / 4;
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const int sl = 4 * ct + g;
        if (ct < nct && sl < nc) {
          const float rs = s_rsc[sl];
          ws.gpart[(((size_t)mm * 4 + cu.q) * ws.max_assign + a0 + sl) * inter + cu.tile * 16 + n] =
              m8_value(acc[ct]) * rs;
        }
      }
    }
    cc = nc_;
    if (it + 1 < i1) cu = item(cc);
  }
  wait_vmcnt_le(0);
}

int moe_grid() { return cu_count() < MOE_MAX_GRID ? cu_count() : MOE_MAX_GRID; }

hipError_t launch_moe_gateup(const sv_moe_desc* d, int R, MoeWs ws, hipStream_t s) {
  (void)R;
  int ca, cq, cd;
  moe8_caps(d, &ca, &cq, &cd);
  const size_t lb = gu_lds_bytes(ca, cq, d->hidden / 256);
  const int nb = d->hidden / 256;
  if (nb == 28)
    hipLaunchKernelGGL(k_gu8f<7>, dim3(moe_grid()), dim3(M8_THREADS), lb, s, expert_ptrs(d), d->inter, ws);
  else if (nb == 32)
    hipLaunchKernelGGL(k_gu8f<8>, dim3(moe_grid()), dim3(M8_THREADS), lb, s, expert_ptrs(d), d->inter, ws);
  else
    hipLaunchKernelGGL(k_gu8, dim3(moe_grid()), dim3(M8_THREADS), lb, s, expert_ptrs(d), nb, d->inter, ws);
  return hipGetLastError();
}

// -------------------------------------------------------------------- down
// The block copies a descriptor's rows of the digit image of the down
// projection's input (k_hdig) into LDS when the descriptor changes.
__device__ __forceinline__ void m8_load_h(const MoeWs& ws, int a0, int nc, int nbd, uint8_t* reg, float* s_rsc) {
  int rows[MOE_WORK_COLS];
#pragma unroll
  for (int c = 0; c < MOE_WORK_COLS; ++c) rows[c] = a0 + min(c, nc - 1);
  m8_load_x(ws.hd, rows, nc, 0, nbd, reg);
  if (threadIdx.x < MOE_WORK_COLS) s_rsc[threadIdx.x] = ws.hd.rsc[rows[threadIdx.x]];
  wait_vmcnt_le(0);
  barrier_lds();
}

__global__ __launch_bounds__(M8_THREADS, 1) void k_dn8(ExpertPtrs P, int hidden, int inter, MoeWs ws) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int TG = hidden / 128, nbd = inter / 256;   // groups of eight 16-row tiles
  const auto work = const_ptr(ws.work_dn);
  const int i0 = const_ptr(ws.blk_dn)[blockIdx.x], i1 = const_ptr(ws.blk_dn)[blockIdx.x + 1];
  if (i0 >= i1) return;
  const int lane = threadIdx.x & 63, w = wave_id();
  const int n = lane & 15, g = lane >> 4;
  uint8_t* ring = lds + (size_t)w * M8_RING * M8_SLOT;
  const uint32_t ring_la = lds_addr(ring);
  float* s_rsc = (float*)(lds + M8_RINGS);   // row scales of the current descriptor's columns
  uint8_t* reg = lds + M8_RINGS + M8_MISC;
  const uint32_t voff = 16u * (uint32_t)lane;
  const size_t tile_bytes = (size_t)M8_CHUNK * nbd;   // one 16-row tile
  auto chunk0 = [&](int dsc, int tg) {
    const int e = work[dsc].expert;
    const uint8_t* mat = e >= 0 ? P.dn + (size_t)e * P.bytes_d : P.sd;
    return mat + (size_t)(tg * 8 + w) * tile_bytes;
  };

  // load cursor: the step at block lkb of tile group ltg of descriptor ld
  int ld = i0 / TG, ltg = i0 - ld * TG, lkb = 0, lleft = i1 - i0, lslot = 0;
  const uint8_t* lp = chunk0(ld, ltg);
  const uint8_t* const pvalid = lp;
  auto issue = [&]() {
    const uint32_t sa = ring_la + (uint32_t)(lslot * M8_SLOT);
    if (lleft > 0) {
      const bool pair = m8_pair(lkb, nbd);
      m8_issue(lp, pair, voff, sa);
      lkb += pair ? 2 : 1;
      lp += pair ? M8_SLOT : M8_CHUNK;
      if (lkb == nbd && --lleft > 0) {
        lkb = 0;
        if (++ltg == TG) {
          ltg = 0;
          ++ld;
        }
        lp = chunk0(ld, ltg);
      }
    } else {
      m8_issue_none(pvalid, voff, sa);
    }
    lslot = lslot == M8_RING - 1 ? 0 : lslot + 1;
  };
  for (int k = 0; k < M8_RING - 1; ++k) issue();

  int cd = i0 / TG, ctg = i0 - cd * TG, cslot = 0, key_d = -1, nc = 1, a0 = 0;
  M8A A = m8_aptr(reg, 1, nbd, lane);
  for (int it = i0; it < i1; ++it) {
    if (cd != key_d) {
      barrier_lds();
      nc = work[cd].ncols;
      a0 = work[cd].a0;
      m8_load_h(ws, a0, nc, nbd, reg, s_rsc);
      key_d = cd;
      A = m8_aptr(reg, nc, nbd, lane);
    }
    const int tile = ctg * 8 + w, nct = (nc + 3) / 4;
    f4_t acc[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) acc[ct] = (f4_t){0.f, 0.f, 0.f, 0.f};
    if (nct == 1) m8_item<1>(ring, cslot, 0, nbd, 0, A, acc, issue);
    else m8_item<2>(ring, cslot, 0, nbd, 0, A, acc, issue);
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const int sl = 4 * ct + g;
      if (ct < nct && sl < nc)
        ws.part[(size_t)(a0 + sl) * hidden + tile * 16 + n] = m8_value(acc[ct]) * s_rsc[sl];
    }
    if (++ctg == TG) {
      ctg = 0;
      ++cd;
    }
  }
  wait_vmcnt_le(0);
}

// The same work for an inter size of NBD = 7 or 8 blocks (four steps per
// tile: patterns A, C), unrolled as in k_gu8f.
template <int NBD>
__global__ __launch_bounds__(M8_THREADS, 1) void k_dn8f(ExpertPtrs P, int hidden, MoeWs ws) {
  using PD = typename std::conditional<NBD == 7, M8PatA, M8PatC>::type;
  extern __shared__ __align__(16) uint8_t lds[];
  const int TG = hidden / 128;
  const auto work = const_ptr(ws.work_dn);
  const int i0 = const_ptr(ws.blk_dn)[blockIdx.x], i1 = const_ptr(ws.blk_dn)[blockIdx.x + 1];
  if (i0 >= i1) return;
  const int lane = threadIdx.x & 63, w = wave_id();
  const int n = lane & 15, g = lane >> 4;
  uint8_t* ring = lds + (size_t)w * M8_RING * M8_SLOT;
  const uint32_t ring_la = lds_addr(ring);
  float* s_rsc = (float*)(lds + M8_RINGS);   // row scales of the current descriptor's columns
  uint8_t* reg = lds + M8_RINGS + M8_MISC;
  const uint32_t voff = 16u * (uint32_t)lane;
  constexpr size_t tile_bytes = (size_t)M8_CHUNK * NBD;   // one 16-row tile
  auto chunk0 = [&](int dsc, int tg) {
    const int e = work[dsc].expert;
    const uint8_t* mat = e >= 0 ? P.dn + (size_t)e * P.bytes_d : P.sd;
    return mat + (size_t)(tg * 8 + w) * tile_bytes;
  };
  auto issue = [&](auto J, const uint8_t* p) {
    constexpr int j = decltype(J)::value;
    const uint32_t sa = ring_la + (uint32_t)(j * M8_SLOT);
    if (p == nullptr) m8_issue_none(P.dn, voff, sa);
    else m8_issue_o(p + PD::off(j), PD::nb(j) == 2, voff, sa);
  };

  int cd = i0 / TG, ctg = i0 - cd * TG, key_d = -1, nc = 1, a0 = 0;
  const uint8_t* cp = chunk0(cd, ctg);
  issue(std::integral_constant<int, 0>(), cp);
  issue(std::integral_constant<int, 1>(), cp);
  issue(std::integral_constant<int, 2>(), cp);
  issue(std::integral_constant<int, 3>(), cp);
  M8A A = m8_aptr(reg, 1, NBD, lane);
  for (int it = i0; it < i1; ++it) {
    int nd_ = cd, ntg = ctg + 1;
    if (ntg == TG) {
      ntg = 0;
      ++nd_;
    }
    const uint8_t* np = it + 1 < i1 ? chunk0(nd_, ntg) : nullptr;
    if (cd != key_d) {
      barrier_lds();
      nc = work[cd].ncols;
      a0 = work[cd].a0;
      m8_load_h(ws, a0, nc, NBD, reg, s_rsc);
      key_d = cd;
      A = m8_aptr(reg, nc, NBD, lane);
    }
    const int tile = ctg * 8 + w, nct = (nc + 3) / 4;
    f4_t acc[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) acc[ct] = (f4_t){0.f, 0.f, 0.f, 0.f};
    auto nx = [&](auto J) { issue(J, np); };
    if (nct == 1) m8_fitem<PD, 1>(ring, A, acc, nx);
    else m8_fitem<PD, 2>(ring, A, acc, nx);
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const int sl = 4 * ct + g;
      if (ct < nct && sl < nc)
        ws.part[(size_t)(a0 + sl) * hidden + tile * 16 + n] = m8_value(acc[ct]) * s_rsc[sl];
    }
    cd = nd_;
    ctg = ntg;
  }
  wait_vmcnt_le(0);
}

hipError_t launch_moe_down(const sv_moe_desc* d, int R, MoeWs ws, hipStream_t s) {
  (void)R;
  int ca, cq, cd;
  moe8_caps(d, &ca, &cq, &cd);
  const size_t lb = dn_lds_bytes(cd, d->inter / 256);
  const int nbd = d->inter / 256;
  if (nbd == 8)
    hipLaunchKernelGGL(k_dn8f<8>, dim3(moe_grid()), dim3(M8_THREADS), lb, s, expert_ptrs(d), d->hidden, ws);
  else if (nbd == 7)
    hipLaunchKernelGGL(k_dn8f<7>, dim3(moe_grid()), dim3(M8_THREADS), lb, s, expert_ptrs(d), d->hidden, ws);
  else
    hipLaunchKernelGGL(k_dn8, dim3(moe_grid()), dim3(M8_THREADS), lb, s, expert_ptrs(d), d->hidden, d->inter, ws);
  return hipGetLastError();
}

// ------------------------------------------------------------ tiled layout
// One thread per (row n, block kb) of each matrix: copies the block's codes,
// nibbles, d and dmin of row n into the chunk of its step (layout in
// specverify.h, sv_q2_tile).
__global__ __launch_bounds__(256) void k_q2_tile(const uint8_t* src, uint8_t* dst, int n_out, int k_in, int parts,
                                                 size_t src_bytes, size_t dst_bytes, long total) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int nb = k_in / 256;
  const long per = (long)n_out * nb;
  const long mat = i / per, x = i - mat * per;
  const int n = (int)(x / nb), kb = (int)(x - (long)n * nb), t = n >> 4, r = n & 15;
  const Q2View W = q2_view(src + (size_t)mat * src_bytes, n_out, k_in);
  int p = 0;
  while (p + 1 < parts && nb * (p + 1) / parts <= kb) ++p;
  const int b0 = nb * p / parts, b1 = nb * (p + 1) / parts;
  int kc, nblk;
  if ((b0 & 1) && kb == b0) {
    kc = kb;
    nblk = 1;
  } else {
    kc = kb & ~1;
    nblk = min(2, b1 - kc);
  }
  const int j = kb - kc;
  uint8_t* ch = dst + (size_t)mat * dst_bytes + (size_t)M8_CHUNK * ((size_t)t * nb + kc);
  const uint4* qs = (const uint4*)(W.qs + ((size_t)n * nb + kb) * 64);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int pc = 4 * j + c, pos = (pc + r) & (4 * nblk - 1);
    *(uint4*)(ch + r * 64 * nblk + 16 * pos) = qs[c];
  }
  {
    const uint4 sc = *(const uint4*)(W.sc + ((size_t)n * nb + kb) * 16);
    const uint32_t w4[4] = {sc.x, sc.y, sc.z, sc.w};
#pragma unroll
    for (int g = 0; g < 4; ++g) *(uint32_t*)(ch + 1024 * nblk + ((j * 4 + g) * 16 + r) * 4) = w4[g];
  }
  *(uint16_t*)(ch + 1280 * nblk + 2 * (r * nblk + j)) = W.d[(size_t)n * nb + kb];
  *(uint16_t*)(ch + 1312 * nblk + 2 * (r * nblk + j)) = W.dm[(size_t)n * nb + kb];
}

hipError_t launch_q2_tile(const void* src, void* dst, int n_out, int k_in, int parts, int count, hipStream_t s) {
  const long total = (long)count * n_out * (k_in / 256);
  const long grid = (total + 255) / 256;
  hipLaunchKernelGGL(k_q2_tile, dim3((unsigned)grid), dim3(256), 0, s, (const uint8_t*)src, (uint8_t*)dst, n_out,
                     k_in, parts, q2_bytes(n_out, k_in), q2_tiled_bytes(n_out, k_in), total);
  return hipGetLastError();
}

}  // namespace sv

// Routed two-bit MoE layer: routing and grouping, the staging of x as byte
// digits, and the weighted combine (the expert kernels are in moe_i8.hip);
// also the one-matrix (PLAIN) form.
//
// Launch sequence of one SwiGLU layer (all on the caller's stream, no host
// sync):
//   k_moe_prep    block 0 routes all rows (top-k on logits, softmax weights;
//                 one wave per row: a DPP maximum and one ballot per slot per
//                 round) and groups (row, slot) pairs by expert so each touched
//                 expert's weights are read once ("MoE gate_up expert dedup",
//                 ds4-on-spark README, introduction), emitting the expert
//                 kernels' descriptors; the other blocks write x as byte digits
//                 (one block per row).
//   k_gu8         gate/up + SwiGLU (moe_i8.hip)
//   k_hdig        the down projection's input rows as digits (one block per
//                 assignment: SwiGLU of the gate/up quarter sums)
//   k_dn8         down projection (moe_i8.hip)
//   k_moe_combine y = fixed-order weighted sum of the per-assignment outputs:
//                 slots 0..k-1, then the shared expert.
#include "sv_digits.h"
#include "sv_internal.h"
#include "sv_q2.h"
#include "sv_stage.h"

namespace sv {

constexpr int LDS_BUDGET = 80 * 1024 - 256;   // one-matrix path: two 512-thread blocks per CU

// Column caps of the expert kernels' descriptors (moe_i8.hip).
void moe8_caps(const sv_moe_desc* d, int* cap_allk, int* cap_quarter, int* cap_down);

// ------------------------------------------------------------ workspace
size_t moe_ws_layout(const sv_moe_desc* d, int R, void* base, MoeWs* out) {
  const bool plain = d->ffn == SV_FFN_PLAIN;
  const int k = plain ? 1 : d->top_k;
  const int has_shared = (!plain && d->s_gate) ? 1 : 0;
  const int max_units = plain ? 1 : (R * k < d->n_experts ? R * k : d->n_experts) + has_shared;
  const int max_assign = plain ? R : R * k + has_shared * R;
  uint8_t* p = (uint8_t*)base;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    void* q = p ? (void*)(p + off) : nullptr;
    off += up256(bytes);
    return q;
  };
  MoeWs w;
  w.meta = (MoeMeta*)take(sizeof(MoeMeta));
  w.unit_expert = (int*)take(sizeof(int) * max_units);
  w.unit_off = (int*)take(sizeof(int) * max_units);
  w.unit_cnt = (int*)take(sizeof(int) * max_units);
  w.arow = (int*)take(sizeof(int) * max_assign);
  w.amap = (int*)take(sizeof(int) * R * (k + 1));
  w.topk_idx = (int*)take(sizeof(int) * R * k);
  w.topk_w = (float*)take(sizeof(float) * R * k);
  w.gpart = (float*)take(plain ? 0 : sizeof(float) * 8 * (size_t)max_assign * d->inter);
  w.part = (float*)take(plain ? 0 : sizeof(float) * (size_t)max_assign * d->hidden);
  // at most one descriptor per unit plus one per further column
  const int max_work = max_units + max_assign;
  w.work_gu = (MoeWork*)take(sizeof(MoeWork) * max_work);
  w.work_dn = (MoeWork*)take(sizeof(MoeWork) * max_work);
  w.blk_gu = (int*)take(sizeof(int) * (MOE_MAX_GRID + 1));
  w.blk_dn = (int*)take(sizeof(int) * (MOE_MAX_GRID + 1));
  void* hd = take(plain ? 0 : xdig_bytes(max_assign, d->inter));
  void* xd = take(plain ? 0 : xdig_bytes(R, d->hidden));
  void* xb = take(plain ? ximg_bytes(R, d->hidden, XL_PERM) : 0);
  const bool q8s = shared_q8(d);
  void* sxb = take(q8s ? ximg_bytes(R, d->hidden, XL_PLAIN) : 0);
  void* shb = take(q8s ? ximg_bytes(R, d->inter, XL_PLAIN) : 0);
  // at most one slice per 512-wide stage of K
  w.sgu = (float*)take(q8s ? sizeof(float) * 2 * (size_t)(d->hidden / 512 + 1) * R * d->inter : 0);
  w.sdn = (float*)take(q8s ? sizeof(float) * (size_t)(d->inter / 512 + 1) * R * d->hidden : 0);
  w.sp_gu = w.sp_dn = 0;
  if (p) {
    if (!plain) w.xd = xdig_carve(xd, R, d->hidden);
    if (!plain) w.hd = xdig_carve(hd, max_assign, d->inter);
    if (plain) w.x_img = ximg_carve(xb, R, d->hidden, XL_PERM);
    if (q8s) {
      w.sx_img = ximg_carve(sxb, R, d->hidden, XL_PLAIN);
      w.sh_img = ximg_carve(shb, R, d->inter, XL_PLAIN);
    }
  }
  w.max_units = max_units;
  w.max_assign = max_assign;
  w.max_work = max_work;
  if (out) *out = w;
  return off;
}

// Largest column group (rows per block) of the one-matrix path whose LDS copy
// fits the budget.
static int col_group(int K, bool use_lo, int R) {
  int cg = XL_MAX_COLS;
  while (cg > 1 && xl_bytes(cg, K, use_lo) > (size_t)LDS_BUDGET) --cg;
  return cg < R ? cg : R;
}

constexpr int DN_THREADS = 512;   // one-matrix path: 8 waves, one 16-row tile each

// ---------------------------------------------------- wave reductions (DPP)
// Reductions to lane 63 on the row-shift / row-broadcast network, then one
// readlane: a few cycles per step instead of an LDS round trip per shuffle.
template <int CTRL, int ROWS>
__device__ inline uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, ROWS, 0xF, false);
}

// (lanes a step does not reach read 0, the identity of the maximum, so the
// move folds into the maximum)
template <int CTRL, int ROWS>
__device__ inline uint32_t dpp0_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xF, false);
}

__device__ inline uint32_t wave_umax32(uint32_t v) {
  v = max(v, dpp0_u32<0x111, 0xF>(v));
  v = max(v, dpp0_u32<0x112, 0xF>(v));
  v = max(v, dpp0_u32<0x114, 0xF>(v));
  v = max(v, dpp0_u32<0x118, 0xF>(v));
  v = max(v, dpp0_u32<0x142, 0xA>(v));
  v = max(v, dpp0_u32<0x143, 0xC>(v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ inline uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Maximum of 64-bit values over the wave: the largest high half, then the
// largest low half among the lanes holding it (two 32-bit reductions, one
// instruction per step each, instead of a 64-bit compare and two selects).
__device__ inline uint64_t wave_umax64(uint64_t v) {
  const uint32_t hi = (uint32_t)(v >> 32), mh = wave_umax32(hi);
  const uint32_t ml = wave_umax32(hi == mh ? (uint32_t)v : 0u);
  return ((uint64_t)mh << 32) | ml;
}

// Sum in a fixed order (run-to-run identical): zeros are shifted in at row
// edges and into the rows a broadcast step leaves alone.
template <int CTRL, int ROWS>
__device__ inline float dpp_add(float x) {
  const int y = __builtin_amdgcn_update_dpp(0, (int)__float_as_uint(x), CTRL, ROWS, 0xF, false);
  return x + __uint_as_float((uint32_t)y);
}

__device__ inline float wave_sum(float x) {
  x = dpp_add<0x111, 0xF>(x);
  x = dpp_add<0x112, 0xF>(x);
  x = dpp_add<0x114, 0xF>(x);
  x = dpp_add<0x118, 0xF>(x);
  x = dpp_add<0x142, 0xA>(x);
  x = dpp_add<0x143, 0xC>(x);
  return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(x), 63));
}

// Inclusive prefix sum over the 64 lanes on the DPP network (row shifts,
// then the row totals broadcast across rows; lanes with no source add 0).
template <int CTRL, int ROWS, int BANKS>
__device__ inline int dpp_z(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWS, BANKS, true);
}
__device__ inline int wave_incl_scan(int x) {
  x += dpp_z<0x111, 0xF, 0xF>(x);   // row_shr:1
  x += dpp_z<0x112, 0xF, 0xF>(x);   // row_shr:2
  x += dpp_z<0x114, 0xF, 0xE>(x);   // row_shr:4
  x += dpp_z<0x118, 0xF, 0xC>(x);   // row_shr:8
  x += dpp_z<0x142, 0xA, 0xF>(x);   // row_bcast:15 into rows 1 and 3
  x += dpp_z<0x143, 0xC, 0xF>(x);   // row_bcast:31 into rows 2 and 3
  return x;
}

// Order-preserving key of a logit: larger logit -> larger key; NaN -> 0, the
// smallest (NaN ranks after every number, as in an ascending sort of -logit).
// Both zeros are one value and get one key (that of +0), so that -0 and +0
// tie and the lower index wins, as for any other pair of equal logits.
__device__ inline uint32_t logit_key(float f) {
  const uint32_t u = __float_as_uint(f);
  if (f != f) return 0u;
  if (f == 0.f) return 0x80000000u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ inline float key_logit(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// ---------------------------------------------------------------- routing
constexpr int PREP_THREADS = 1024;

// One wave: top-k of one row of E logits (E <= 64 * PER), by logit, ties to
// the lower index; weights = softmax probability over all E.  Every expert is
// one 64-bit value, its logit's key above the complement of its index, so the
// order of these values is the order of choice and no two are equal (slots
// past E hold 0, below every expert).  Each lane sorts its PER values; in each
// of k rounds the largest head over the wave is the next choice and the lane
// holding it moves to its next value.
template <int PER>
__device__ void route_row(const float* logits, int r, int E, int k, int* s_idx, int32_t* idx_out,
                          float* w_out, MoeWs ws) {
  const int lane = threadIdx.x & 63;
  float v[PER];
  uint64_t c[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? logits[(size_t)r * E + e] : -INFINITY;
    c[i] = e < E ? ((uint64_t)logit_key(v[i]) << 32) | (uint32_t)~(uint32_t)e : 0ull;
  }
#pragma unroll
  for (int i = 1; i < PER; ++i)
#pragma unroll
    for (int j = i; j > 0; --j) {
      const uint64_t hi = umax64(c[j - 1], c[j]), lo = c[j - 1] ^ c[j] ^ hi;
      c[j - 1] = hi;
      c[j] = lo;
    }
  // lane s keeps the s-th choice; all k are written together afterwards
  uint64_t mine = 0, first = 0;
  for (int s = 0; s < k; ++s) {
    const uint64_t g = wave_umax64(c[0]);
    if (s == 0) first = g;
    if (c[0] == g) {
#pragma unroll
      for (int j = 0; j + 1 < PER; ++j) c[j] = c[j + 1];
      c[PER - 1] = 0;
    }
    if (lane == s) mine = g;
  }
  const float mx = key_logit((uint32_t)(first >> 32));   // the largest logit
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i)
    if (lane + 64 * i < E) sum += expf(v[i] - mx);
  sum = wave_sum(sum);
  if (lane < k) {
    const int my_idx = (int)~(uint32_t)mine;
    const float w = expf(key_logit((uint32_t)(mine >> 32)) - mx) / sum;
    s_idx[r * k + lane] = my_idx;
    ws.topk_idx[r * k + lane] = my_idx;
    ws.topk_w[r * k + lane] = w;
    if (idx_out) idx_out[r * k + lane] = my_idx;
    if (w_out) w_out[r * k + lane] = w;
  }
}

// Block 0 of the prep kernel: top-k of every row, then grouping.
// Descriptors of one expert kernel (wave 0): each unit's assignments in
// column groups.  Gate/up: a unit of at most cap_allk rows is one MOE_ALLK
// descriptor, a larger one is cut into MOE_QUARTER descriptors of at most
// cap_big rows; down: groups of at most cap_big rows, typed like the unit's
// gate/up work.  Then the item ranges of the kernel's G persistent blocks:
// every descriptor costs MOE_SWITCH_* and then has `items` items, each costing
// MOE_COST_1 (at most four rows) or MOE_COST_2_*; block b starts at the first
// item whose cost offset is at least floor(C b / G) (C the total cost), so the
// ranges are contiguous, cover every item once and carry about equal cost
// (a block whose range crosses into another descriptor takes fewer items).
__device__ void emit_work(const int* s_uexp, const int* s_uoff, const int* s_ucnt, int nu,
                          const int* s_arow, bool gateup, int cap_allk, int cap_big, int items, int G,
                          MoeWork* work, int* n_work, int* blk, int* s_cost) {
  const int lane = threadIdx.x & 63;
  int base = 0;
  for (int u0 = 0; u0 < nu; u0 += 64) {
    const int u = u0 + lane;
    const int cnt = u < nu ? s_ucnt[u] : 0;
    const int type = cnt <= cap_allk ? MOE_ALLK : MOE_QUARTER;
    const int grp = (gateup && type == MOE_ALLK) ? cap_allk : cap_big;
    const int ng = u < nu ? (cnt + grp - 1) / grp : 0;
    const int incl = wave_incl_scan(ng);
    for (int j = 0; j < ng; ++j) {
      MoeWork w;
      w.expert = s_uexp[u];
      w.a0 = s_uoff[u] + j * grp;
      w.ncols = min(grp, cnt - j * grp);
      w.type = type;
#pragma unroll
      for (int c = 0; c < MOE_WORK_COLS; ++c) w.rows[c] = c < w.ncols ? s_arow[w.a0 + c] : 0;
      work[base + incl - ng + j] = w;
      s_cost[base + incl - ng + j + 1] = w.ncols > 4 ? (gateup ? MOE_COST_2_GU : MOE_COST_2_DN) : MOE_COST_1;
    }
    base += __builtin_amdgcn_readlane(incl, 63);
  }
  const int nd = base;
  if (lane == 0) *n_work = nd;
  // s_cost[d] becomes the cost offset of descriptor d (its change cost sw,
  // then its items)
  const int sw = gateup ? MOE_SWITCH_GU : MOE_SWITCH_DN;
  if (lane == 0) s_cost[0] = 0;
  __builtin_amdgcn_s_waitcnt(0xC07F);
  int run = 0;
  for (int d0 = 1; d0 <= nd; d0 += 64) {
    const int d = d0 + lane;
    const int c = d <= nd ? s_cost[d] * items + sw : 0;
    const int incl = wave_incl_scan(c);
    if (d <= nd) s_cost[d] = run + incl;
    run += __builtin_amdgcn_readlane(incl, 63);
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);
  const int C = run;
  if (C == 0) {
    for (int b = lane; b <= G; b += 64) blk[b] = 0;
    return;
  }
  // Block b starts at the first item whose cost offset is at least
  // c = floor(C b / G): in the descriptor d with s_cost[d] <= c < s_cost[d+1],
  // at item ceil(max(0, c - s_cost[d] - sw) / w), w the descriptor's cost per
  // item (an item past the descriptor's last is the next one's first).  Every
  // product here is below 2^53, and a quotient that is not an integer is at
  // least 1/C away from one, so the fp64 floors and ceilings are exact.
  const double dG = (double)G, dC = (double)C;
  auto first = [&](int c, int P0, int w) {
    const int t = c - P0 - sw;
    return t <= 0 ? 0 : (t + w - 1) / w;
  };
  if (nd < 16) {
    // few descriptors, many blocks each: lane l takes blocks l, l + 64, ...
    // and finds its descriptor by bisection (the offsets increase strictly)
    for (int b = lane; b < G; b += 64) {
      const int c = (int)floor(dC * (double)b / dG);
      int lo = 0, hi = nd - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_cost[mid] <= c) lo = mid;
        else hi = mid - 1;
      }
      const int P0 = s_cost[lo], w = (s_cost[lo + 1] - P0 - sw) / items;
      blk[b] = lo * items + first(c, P0, w);
    }
  } else {
    // lane l takes descriptors l, l + 64, ... and writes the blocks that
    // start in them, b in [ceil(s_cost[d] G / C), ceil(s_cost[d+1] G / C));
    // after the first, c steps by C = qG G + rG: c(b + 1) = c(b) + qG, plus
    // one when the remainder C b - c G passes G
    const int qG = C / G, rG = C - qG * G;
    for (int d = lane; d < nd; d += 64) {
      const int P0 = s_cost[d], P1 = s_cost[d + 1], w = (P1 - P0 - sw) / items;
      const int b0 = (int)ceil((double)P0 * dG / dC), b1 = (int)ceil((double)P1 * dG / dC);
      int c = (int)floor(dC * (double)b0 / dG);
      int r = (int)((long long)C * b0 - (long long)c * G);
      for (int b = b0; b < b1; ++b) {
        blk[b] = d * items + first(c, P0, w);
        c += qG;
        r += rG;
        if (r >= G) {
          ++c;
          r -= G;
        }
      }
    }
  }
  if (lane == 0) blk[G] = nd * items;
}

// has_shared: the layer has a shared expert (its R assignments follow the
// routed ones); shared_work: the two-bit expert kernels compute it (not when
// it is eight-bit).
__device__ void route_and_group(const float* logits, int R, int E, int k, int has_shared, int shared_work,
                                int cap_allk, int cap_quarter, int cap_down, int items_gu, int items_dn, int G,
                                int32_t* idx_out, float* w_out, MoeWs ws) {
  // cost offsets of the descriptors (at most one per unit plus one per further row)
  __shared__ int s_cost_gu[SV_MAX_EXPERTS + 2 + SV_MAX_ROWS * (SV_MAX_TOPK + 1)];
  __shared__ int s_cost_dn[SV_MAX_EXPERTS + 2 + SV_MAX_ROWS * (SV_MAX_TOPK + 1)];
  __shared__ int s_idx[SV_MAX_ROWS * SV_MAX_TOPK];
  __shared__ unsigned long long s_rmask[SV_MAX_EXPERTS];   // rows that chose expert e (R <= 64)
  __shared__ int eoff[SV_MAX_EXPERTS];
  __shared__ int s_uexp[SV_MAX_EXPERTS + 1], s_uoff[SV_MAX_EXPERTS + 1], s_ucnt[SV_MAX_EXPERTS + 1];
  __shared__ int s_arow[SV_MAX_ROWS * (SV_MAX_TOPK + 1)];
  __shared__ int s_nu;
  const int tid = threadIdx.x, lane = tid & 63, wv = wave_id();
  constexpr int NW = PREP_THREADS / 64;
  for (int e = tid; e < E; e += PREP_THREADS) s_rmask[e] = 0ull;
  if (logits == nullptr) {  // one expert, no router: weight 1
    for (int i = tid; i < R * k; i += PREP_THREADS) {
      s_idx[i] = 0;
      ws.topk_idx[i] = 0;
      ws.topk_w[i] = 1.f;
      if (idx_out) idx_out[i] = 0;
      if (w_out) w_out[i] = 1.f;
    }
  } else {
    for (int r = wv; r < R; r += NW) {
      if (E <= 64) route_row<1>(logits, r, E, k, s_idx, idx_out, w_out, ws);
      else if (E <= 128) route_row<2>(logits, r, E, k, s_idx, idx_out, w_out, ws);
      else if (E <= 256) route_row<4>(logits, r, E, k, s_idx, idx_out, w_out, ws);
      else if (E <= 512) route_row<8>(logits, r, E, k, s_idx, idx_out, w_out, ws);
      else route_row<16>(logits, r, E, k, s_idx, idx_out, w_out, ws);
    }
  }
  __syncthreads();
  for (int i = tid; i < R * k; i += PREP_THREADS) atomicOr(&s_rmask[s_idx[i]], 1ull << (i / k));
  __syncthreads();
  if (wv == 0) {  // touched experts in ascending order -> units, assignment offsets
    int base_u = 0, base_a = 0;
    for (int c0 = 0; c0 < E; c0 += 64) {
      const int e = c0 + lane;
      const int ce = e < E ? __popcll(s_rmask[e]) : 0;
      const int fu = wave_incl_scan(ce > 0 ? 1 : 0), fa = wave_incl_scan(ce);
      const int u = base_u + fu - (ce > 0 ? 1 : 0);
      const int a = base_a + fa - ce;
      if (e < E) eoff[e] = a;
      if (ce > 0) {
        ws.unit_expert[u] = e;
        ws.unit_off[u] = a;
        ws.unit_cnt[u] = ce;
        s_uexp[u] = e;
        s_uoff[u] = a;
        s_ucnt[u] = ce;
      }
      base_u += __builtin_amdgcn_readlane(fu, 63);
      base_a += __builtin_amdgcn_readlane(fa, 63);
    }
    if (lane == 0) s_nu = base_u;
  }
  __syncthreads();
  const int nu = s_nu;
  for (int i = tid; i < R * k; i += PREP_THREADS) {
    const int r = i / k, s = i - r * k, e = s_idx[i];
    // rows before r that chose e (each row picks an expert at most once)
    const int rank = __popcll(s_rmask[e] & ((1ull << r) - 1ull));
    const int a = eoff[e] + rank;
    ws.arow[a] = r;
    s_arow[a] = r;
    ws.amap[r * (k + 1) + s] = a;
  }
  if (has_shared) {
    for (int r = tid; r < R; r += PREP_THREADS) {
      ws.arow[R * k + r] = r;
      s_arow[R * k + r] = r;
      ws.amap[r * (k + 1) + k] = R * k + r;
    }
    if (tid == 0) {
      ws.unit_expert[nu] = -1;
      ws.unit_off[nu] = R * k;
      ws.unit_cnt[nu] = R;
      s_uexp[nu] = -1;
      s_uoff[nu] = R * k;
      s_ucnt[nu] = R;
    }
  }
  if (tid == 0) {
    ws.meta->n_units = nu + has_shared;
    ws.meta->n_assign = R * k + has_shared * R;
  }
  __syncthreads();
  const int nwu = nu + (has_shared && shared_work ? 1 : 0);   // units the expert kernels compute
  if (wv == 0) emit_work(s_uexp, s_uoff, s_ucnt, nwu, s_arow, true, cap_allk, cap_quarter, items_gu,
                         G, ws.work_gu, &ws.meta->n_work_gu, ws.blk_gu, s_cost_gu);
  if (wv == 1) emit_work(s_uexp, s_uoff, s_ucnt, nwu, s_arow, false, cap_allk, cap_down, items_dn,
                         G, ws.work_dn, &ws.meta->n_work_dn, ws.blk_dn, s_cost_dn);
}

// ------------------------------------------------------------ rows as digits
// One block per row: thread t converts sub-blocks t, t + PREP_THREADS, ...
// (16 values each, loaded once by load(sb, v)), after a block-wide maximum of
// the row.
template <typename Load>
__device__ void stage_row_digits(int row, XDig xd, Load load) {
  __shared__ uint32_t s_max;
  __shared__ int s_bad;
  const int K = xd.K, nsb = K / 16, tid = threadIdx.x;
  constexpr int PER = (16384 / 16 + PREP_THREADS - 1) / PREP_THREADS;
  float v[PER][16];
  float mx = 0.f;
  int bad = 0;
  if (tid == 0) {
    s_max = 0u;
    s_bad = 0;
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int sb = tid + PREP_THREADS * i;
#pragma unroll
    for (int e = 0; e < 16; ++e) v[i][e] = 0.f;
    if (sb < nsb) {
      load(sb, v[i]);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float a = fabsf(v[i][e]);
        bad |= !(a <= 3.402823466e38f);
        mx = fmaxf(mx, a);
      }
    }
  }
  __syncthreads();
  mx = wave_allreduce(mx, [](float a, float b) { return fmaxf(a, b); });
  if ((tid & 63) == 0) atomicMax(&s_max, __float_as_uint(mx));
  if (__any(bad) && (tid & 63) == 0) s_bad = 1;
  __syncthreads();
  const bool rbad = s_bad != 0;
  const int s = rbad ? 0 : digit_exponent(__uint_as_float(s_max));
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int sb = tid + PREP_THREADS * i;
    if (sb >= nsb) continue;
    uint4 pl[NDIG];
    int sums[NDIG];
    subblock_digits(v[i], s, rbad, pl, sums);
#pragma unroll
    for (int p = 0; p < NDIG; ++p) {
      *(uint4*)(xd.dig + ((size_t)row * NDIG + p) * K + subblock_offset(sb)) = pl[p];
      xd.sx[((size_t)row * NDIG + p) * nsb + sb] = (_Float16)(float)sums[p];
    }
  }
  if (tid == 0) xd.rsc[row] = rbad ? __builtin_nanf("") : ldexpf(1.f, -s);
}

// Row `row` of x (bf16 or fp32) as digits.
template <int DT>
__device__ void stage_digits(const void* x, int row, XDig xd) {
  const int K = xd.K;
  stage_row_digits(row, xd, [&](int sb, float (&v)[16]) {
    const size_t o = (size_t)row * K + 16 * sb;
    if (DT == SV_BF16) {
      const uint4 a = *(const uint4*)((const uint16_t*)x + o);
      const uint4 b = *(const uint4*)((const uint16_t*)x + o + 8);
      const uint32_t u[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        v[2 * j] = __uint_as_float(u[j] << 16);
        v[2 * j + 1] = __uint_as_float(u[j] & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 f = *(const float4*)((const float*)x + o + 4 * j);
        v[4 * j] = f.x;
        v[4 * j + 1] = f.y;
        v[4 * j + 2] = f.z;
        v[4 * j + 3] = f.w;
      }
    }
  });
}

// The down projection's input of assignment a as digits: silu(sum of the
// gate quarters) * (sum of the up quarters), quarters summed in order (the
// SwiGLU of the gate/up kernels' quarter sums).  One block per assignment:
// every thread first forms four of the row's values into LDS (so the loads
// and the SwiGLU are spread over the whole block), then the row is turned
// into digits one sub-block per thread.
__global__ __launch_bounds__(PREP_THREADS) void k_hdig(MoeWs ws, int inter) {
  extern __shared__ __align__(16) float s_h[];   // [inter]
  const int a = blockIdx.x;
  const size_t qs = (size_t)ws.max_assign * inter, o = (size_t)a * inter;
  for (int i = threadIdx.x; 4 * i < inter; i += PREP_THREADS) {
    float4 gq[4], uq[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      gq[q] = *(const float4*)(ws.gpart + (size_t)q * qs + o + 4 * i);
      uq[q] = *(const float4*)(ws.gpart + (size_t)(4 + q) * qs + o + 4 * i);
    }
    float4 h;
    h.x = silu_mul(((gq[0].x + gq[1].x) + gq[2].x) + gq[3].x, ((uq[0].x + uq[1].x) + uq[2].x) + uq[3].x);
    h.y = silu_mul(((gq[0].y + gq[1].y) + gq[2].y) + gq[3].y, ((uq[0].y + uq[1].y) + uq[2].y) + uq[3].y);
    h.z = silu_mul(((gq[0].z + gq[1].z) + gq[2].z) + gq[3].z, ((uq[0].z + uq[1].z) + uq[2].z) + uq[3].z);
    h.w = silu_mul(((gq[0].w + gq[1].w) + gq[2].w) + gq[3].w, ((uq[0].w + uq[1].w) + uq[2].w) + uq[3].w);
    *(float4*)(s_h + 4 * i) = h;
  }
  __syncthreads();
  stage_row_digits(a, ws.hd, [&](int sb, float (&v)[16]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 h = *(const float4*)(s_h + 16 * sb + 4 * j);
      v[4 * j] = h.x;
      v[4 * j + 1] = h.y;
      v[4 * j + 2] = h.z;
      v[4 * j + 3] = h.w;
    }
  });
}

hipError_t launch_hdig(const sv_moe_desc* d, int R, MoeWs ws, hipStream_t s) {
  // the eight-bit shared expert's assignments (the last R) have no quarter sums
  const int na = shared_q8(d) ? ws.max_assign - R : ws.max_assign;
  hipLaunchKernelGGL(k_hdig, dim3(na), dim3(PREP_THREADS), (size_t)d->inter * sizeof(float), s, ws, d->inter);
  return hipGetLastError();
}

template <int DT>
__global__ __launch_bounds__(PREP_THREADS) void k_moe_prep(const float* logits, int R, int E, int k,
                                                           int has_shared, int shared_work, int cap_allk,
                                                           int cap_quarter,
                                                           int cap_down, int items_gu, int items_dn, int G,
                                                           int32_t* idx_out, float* w_out, const void* x,
                                                           MoeWs ws) {
  if (blockIdx.x == 0) {
    route_and_group(logits, R, E, k, has_shared, shared_work, cap_allk, cap_quarter, cap_down, items_gu, items_dn,
                    G, idx_out,
                    w_out, ws);
  } else {
    stage_digits<DT>(x, blockIdx.x - 1, ws.xd);   // one block per row
  }
}

hipError_t launch_moe_prep(const sv_moe_desc* d, int R, const float* router_logits,
                           const void* x, int x_dtype, int32_t* topk_idx_out,
                           float* topk_w_out, MoeWs ws, hipStream_t s) {
  const int has_shared = d->s_gate ? 1 : 0, shared_work = shared_q8(d) ? 0 : 1;
  const dim3 grid(1 + R);
  int ca, cq, cd;
  moe8_caps(d, &ca, &cq, &cd);
  const int items_gu = d->inter / 16, items_dn = d->hidden / 128, G = moe_grid();
  if (x_dtype == SV_BF16)
    hipLaunchKernelGGL(k_moe_prep<SV_BF16>, grid, dim3(PREP_THREADS), 0, s, router_logits, R, d->n_experts,
                       d->top_k, has_shared, shared_work, ca, cq, cd, items_gu, items_dn, G, topk_idx_out,
                       topk_w_out, x, ws);
  else
    hipLaunchKernelGGL(k_moe_prep<SV_F32>, grid, dim3(PREP_THREADS), 0, s, router_logits, R, d->n_experts,
                       d->top_k, has_shared, shared_work, ca, cq, cd, items_gu, items_dn, G, topk_idx_out,
                       topk_w_out, x, ws);
  return hipGetLastError();
}

// ------------------------------------------------ one-matrix path staging
// Activation rows are copied into LDS in 1 KB pieces.
__host__ __device__ inline int xl_pieces_per_row(int K, bool use_lo) {
  return ((2 * K + 1023) / 1024) * (use_lo ? 2 : 1) + (K / 4 + 1023) / 1024;
}

struct XLw {   // writable view of the LDS rows
  _Float16 *hi, *lo, *sx;
  float* rsc;
  int K, rs, sxs;
};

__device__ inline XLw xl_make(uint8_t* lds, int ncols, int K, bool use_lo) {
  XLw w;
  xl_carve<_Float16>((_Float16*)lds, ncols, K, use_lo, w.hi, w.lo, w.sx, w.rsc);
  w.K = K;
  w.rs = xl_rs(K);
  w.sxs = K / 8;
  return w;
}

__device__ inline XL xl_view(const XLw& w) {
  XL x;
  x.hi = w.hi;
  x.lo = w.lo;
  x.sx = w.sx;
  x.rsc = w.rsc;
  x.rs = w.rs;
  x.sxs = w.sxs;
  return x;
}

// Prepared image rows are copied into LDS with global-to-LDS loads (no
// registers), issued before the weight loads; each wave then waits for its own
// copies with an explicit vmcnt (they are older than every weight load) and
// the block meets at a barrier.  The copy is written as inline assembly: when
// the compiler sees an outstanding global-to-LDS load it waits for every
// vector load before the next use, which would serialise the weight stream.
// Source, destination and length of piece j of column c (image row r).
struct XLPiece {
  const uint8_t* src;
  uint32_t la;      // LDS byte address of the destination
  int bytes;
};

// LDS byte address of a generic pointer into the LDS aperture.  Each branch of
// xl_piece converts its own pointer, so that no select of generic LDS
// pointers reaches the conversion (the backend fails on that form).
__device__ __forceinline__ uint32_t lds_la(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}

__device__ __forceinline__ XLPiece xl_piece(const XImg& img, const XLw& L, int r, int c, int j,
                                            bool use_lo) {
  const int K = L.K, prow = (2 * K + 1023) / 1024;
  XLPiece p;
  if (j < prow) {
    p.src = (const uint8_t*)(img.hi + (size_t)r * K) + 1024 * j;
    p.la = lds_la(L.hi + (size_t)c * L.rs) + 1024 * j;
    p.bytes = 2 * K - 1024 * j;
  } else if (use_lo && j < 2 * prow) {
    const int jj = j - prow;
    p.src = (const uint8_t*)(img.lo + (size_t)r * K) + 1024 * jj;
    p.la = lds_la(L.lo + (size_t)c * L.rs) + 1024 * jj;
    p.bytes = 2 * K - 1024 * jj;
  } else {
    const int jj = j - prow * (use_lo ? 2 : 1);
    p.src = (const uint8_t*)(img.sx + (size_t)r * (K / 8)) + 1024 * jj;
    p.la = lds_la(L.sx + (size_t)c * L.sxs) + 1024 * jj;
    p.bytes = K / 4 - 1024 * jj;
  }
  p.la = __builtin_amdgcn_readfirstlane(p.la);
  return p;
}

// Row c of the block is image row rows[c] (rows in global memory, read with
// wave-uniform scalar loads), or row0 + c when rows is null.
__device__ __forceinline__ int xl_row(const int* rows, int row0, int c) {
  return rows ? const_ptr(rows)[c] : row0 + c;
}

// Lane i copies bytes [16 i, 16 i + 16) of a 1 KB piece from global memory to
// LDS (lanes past `bytes` skip); la is the wave-uniform LDS byte address.
__device__ __forceinline__ void dma_piece(const uint8_t* src, uint32_t la, int bytes) {
  const int lane = threadIdx.x & 63;
  if (16 * lane < bytes)
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(src + 16 * lane), "s"(la) : "memory", "m0");
}

__device__ __forceinline__ void xl_img_dma(const XImg& img, const int* rows, int row0, int ncols,
                                           bool use_lo, const XLw& L) {
  const int wv = wave_id(), nw = blockDim.x >> 6;
  const int per_c = xl_pieces_per_row(L.K, use_lo), total = ncols * per_c;
  for (int q = wv; q < total; q += nw) {
    const int c = __builtin_amdgcn_readfirstlane(q / per_c);   // wave-uniform: scalar row reads
    const XLPiece p = xl_piece(img, L, xl_row(rows, row0, c), c, q - c * per_c, use_lo);
    dma_piece(p.src, p.la, p.bytes);
  }
}

// --------------------------------------------------------------- combine
// y[r, n] = sum_{s<k} w[r, s] * part[a(r, s), n] (+ part[a(r, shared), n]), in slot order.
// SQ8: the shared expert is eight-bit and its output the sum of its
// sdn_parts down slices (in order); otherwise it is in ws.part like the
// routed ones.
template <bool SQ8>
__global__ __launch_bounds__(256) void k_moe_combine(int hidden, int k, int has_shared, int sdn_parts, int R,
                                                     MoeWs ws, float* y) {
  __shared__ int s_a[SV_MAX_TOPK + 1];
  __shared__ float s_w[SV_MAX_TOPK];
  const int r = blockIdx.y, tid = threadIdx.x;
  if (tid <= k) s_a[tid] = ws.amap[r * (k + 1) + tid];
  if (tid < k) s_w[tid] = ws.topk_w[r * k + tid];
  __syncthreads();
  const int n4 = blockIdx.x * 256 + tid;   // 4 outputs per thread
  if (4 * n4 >= hidden) return;
  const int ns = k + has_shared;
  float4 v[SV_MAX_TOPK + 1];
#pragma unroll
  for (int s = 0; s <= SV_MAX_TOPK; ++s)
    if (s < (SQ8 ? k : ns)) v[s] = *(const float4*)(ws.part + (size_t)s_a[s] * hidden + 4 * n4);
  if (SQ8) {
    const float* sp = ws.sdn + (size_t)r * hidden + 4 * n4;
    float4 a = *(const float4*)sp;
    for (int p = 1; p < sdn_parts; ++p) {
      const float4 b = *(const float4*)(sp + (size_t)p * R * hidden);
      a.x += b.x;
      a.y += b.y;
      a.z += b.z;
      a.w += b.w;
    }
    v[k] = a;
  }
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int s = 0; s <= SV_MAX_TOPK; ++s) {
    if (s < k) {
      acc.x = fmaf(s_w[s], v[s].x, acc.x);
      acc.y = fmaf(s_w[s], v[s].y, acc.y);
      acc.z = fmaf(s_w[s], v[s].z, acc.z);
      acc.w = fmaf(s_w[s], v[s].w, acc.w);
    } else if (s == k && has_shared) {   // the shared expert last, weight 1
      acc.x += v[s].x;
      acc.y += v[s].y;
      acc.z += v[s].z;
      acc.w += v[s].w;
    }
  }
  *(float4*)(y + (size_t)r * hidden + 4 * n4) = acc;
}

hipError_t launch_moe_combine(const sv_moe_desc* d, int R, MoeWs ws, float* y, hipStream_t s) {
  const dim3 grid((d->hidden / 4 + 255) / 256, R);
  if (shared_q8(d))
    hipLaunchKernelGGL(k_moe_combine<true>, grid, dim3(256), 0, s, d->hidden, d->top_k, 1,
                       ws.sp_dn > 0 ? ws.sp_dn : 1, R, ws, y);
  else
    hipLaunchKernelGGL(k_moe_combine<false>, grid, dim3(256), 0, s, d->hidden, d->top_k, d->s_gate ? 1 : 0, 0, R,
                       ws, y);
  return hipGetLastError();
}

// ------------------------------------------------ eight-bit shared expert
// The products run on the vocabulary head's kernel split over K (the shared
// expert's 2048-row matrices alone would occupy few compute units), or
// unsplit where the split form does not take the shape (one slice).
void plan_shared_q8(const sv_moe_desc* d, int R, int x_dtype, MoeWs* ws) {
  ws->sp_gu = q8_split_parts(d->inter, d->hidden, R, x_dtype == SV_F32, 2);
  ws->sp_dn = q8_split_parts(d->hidden, d->inter, R, true, 1);
}

// Stages h = silu(g) * u of the shared expert for the down product, g and u
// summed over their K slices in order as they are loaded.
__global__ __launch_bounds__(256) void k_stage_swiglu(const float* gu, int parts, int R, XImg img) {
  __shared__ int sh[8];
  const int I = img.K, row = blockIdx.x;
  const size_t ps = (size_t)R * I;
  const float* g = gu + (size_t)row * I;
  const float* u = g + (size_t)parts * ps;
  stage_row_l<256>(row, XL_PLAIN, img, sh, [&](int k, float* v) {
    float4 a = *(const float4*)(g + k), b = *(const float4*)(u + k);
    for (int p = 1; p < parts; ++p) {
      const float4 a2 = *(const float4*)(g + p * ps + k), b2 = *(const float4*)(u + p * ps + k);
      a.x += a2.x; a.y += a2.y; a.z += a2.z; a.w += a2.w;
      b.x += b2.x; b.y += b2.y; b.z += b2.z; b.w += b2.w;
    }
    v[0] = silu_mul(a.x, b.x);
    v[1] = silu_mul(a.y, b.y);
    v[2] = silu_mul(a.z, b.z);
    v[3] = silu_mul(a.w, b.w);
  });
}

hipError_t launch_shared_q8(const sv_moe_desc* d, int R, const void* x, int x_dtype, MoeWs ws,
                            hipStream_t s) {
  const int H = d->hidden, I = d->inter;
  hipError_t e = launch_stage(x, x_dtype, R, H, XL_PLAIN, nullptr, ws.sx_img, s);
  if (e != hipSuccess) return e;
  const bool lo = x_dtype == SV_F32;   // bf16 rows are exact in the fp16 high part
  int pg = ws.sp_gu;
  if (pg > 0) {
    e = launch_q8_split(d->s_gate, d->s_up, I, H, R, lo, ws.sx_img, ws.sgu, s);
  } else {
    pg = 1;
    if ((e = launch_q8_lmhead(d->s_gate, I, H, R, lo, ws.sx_img, ws.sgu, s)) != hipSuccess) return e;
    e = launch_q8_lmhead(d->s_up, I, H, R, lo, ws.sx_img, ws.sgu + (size_t)R * I, s);
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_stage_swiglu, dim3(R), dim3(256), 0, s, ws.sgu, pg, R, ws.sh_img);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ws.sp_dn > 0) return launch_q8_split(d->s_down, nullptr, H, I, R, true, ws.sh_img, ws.sdn, s);
  return launch_q8_lmhead(d->s_down, H, I, R, true, ws.sh_img, ws.sdn, s);
}

// ----------------------------------------------------------------- plain
// y[R, n_out] = W x for one two-bit matrix: 8 waves of one 16-row tile each
// over all of K, the block's rows (a group of up to CG of the R rows) in LDS.
template <bool USE_LO, bool WIDE_D>
__global__ __launch_bounds__(DN_THREADS, 4) void k_q2_plain(const uint8_t* w, int n_out, int k_in,
                                                            int R, int CG, XImg img, float* y) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int c0 = blockIdx.z * CG;
  const int ncols = min(CG, R - c0);
  const int tid = threadIdx.x, lane = tid & 63, wv = wave_id();
  const int nl = lane & 15, g = lane >> 4;
  const int n = (blockIdx.x * 8 + wv) * 16 + nl;
  const int nld = n < n_out ? n : n_out - 1;   // ragged tail: load a valid row, drop the result
  const Q2View W = q2_view(w, n_out, k_in);
  const XLw L = xl_make(lds, ncols, k_in, USE_LO);
  f4_t acc = {0.f, 0.f, 0.f, 0.f};
  auto issue = [&]() { xl_img_dma(img, nullptr, c0, ncols, USE_LO, L); };
  auto sync = [&](int nload) {
    wait_vmcnt_le(nload);
    barrier_keep_loads();
  };
  q2_range_staged<WIDE_D, USE_LO>(W, nld, 0, k_in / 256, xl_view(L), min(nl, ncols - 1), lane, acc,
                                  issue, sync);
  if (n >= n_out) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = 4 * g + i;
    if (c < ncols) y[(size_t)(c0 + c) * n_out + n] = acc[i] * img.rscale[c0 + c];
  }
}

hipError_t launch_q2_plain(const sv_moe_desc* d, int R, bool use_lo, MoeWs ws, float* y,
                           hipStream_t s) {
  const int CG = col_group(d->hidden, use_lo, R);
  const int tiles = (d->inter + 15) / 16;
  const dim3 grid((tiles + 7) / 8, 1, (R + CG - 1) / CG);
  const size_t lb = xl_bytes(CG, d->hidden, use_lo);
  const bool wide = q2_wide_d(d->hidden / 256);
  const uint8_t* w = (const uint8_t*)d->w_gate;
#define SV_PL(LO, WD)                                                                          \
  hipLaunchKernelGGL((k_q2_plain<LO, WD>), grid, dim3(DN_THREADS), lb, s, w, d->inter, d->hidden, \
                     R, CG, ws.x_img, y)
  if (use_lo) {
    if (wide) SV_PL(true, true); else SV_PL(true, false);
  } else {
    if (wide) SV_PL(false, true); else SV_PL(false, false);
  }
#undef SV_PL
  return hipGetLastError();
}

}  // namespace sv

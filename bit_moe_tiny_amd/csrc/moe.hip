// Routed two-bit MoE layer: routing + grouping, fused gate/up/SwiGLU, down
// projection with a fixed-order weighted combine, and the one-matrix form.
//
// Launch sequence of one layer (all on the caller's stream, no host sync):
//   k_moe_prep    block 0 routes all rows (top-k on logits, softmax weights;
//                 one wave per row: a DPP maximum and one ballot per slot per
//                 round)
//                 and groups (row, slot) pairs by expert so each touched
//                 expert's weights are read once ("MoE gate_up expert dedup",
//                 ds4-on-spark README, introduction); the other blocks stage x
//                 into the fp16 image the two-bit kernels read.
//   k_q2_gateup_p persistent, 2 blocks per CU of 8 waves (gate and up x 4
//                 parts of hidden), each block a contiguous range of (work
//                 item, 16-row tile of inter) with the next item's weight loads
//                 in flight; the partial sums meet in LDS and one wave applies
//                 SwiGLU ("fused gate+up+swiglu MoE decode", 1x Spark tuned
//                 DSpark thread, Q&A answer 3).  h is kept in fp32, and each
//                 h row's largest magnitude is raised by atomic max (the
//                 down projection's scale; k_moe_prep clears it).
//   k_q2_gateup   the same per (tile, work item) block, for shapes the
//                 persistent kernel does not take.
//   k_q2_down     grid (128-row group of hidden, unit, column group of at
//                 most 4 rows), 8 waves of one 16-row tile over all of inter,
//                 on the int8 matrix cores: the block converts its h rows into
//                 four fixed-point byte digits each (four tile columns per
//                 row; the scale from the row's recorded largest magnitude)
//                 in LDS, the weights enter as the bytes sc * q, every block
//                 product is exact; per-assignment outputs go to the
//                 workspace.
//   k_moe_combine y = fixed-order weighted sum of the per-assignment outputs:
//                 slots 0..k-1, then the shared expert.
// Blocks never wait on each other inside a kernel: on a part whose L2 is split
// across dies, a device-wide fence per block would cost far more than the
// extra launch.
#include "sv_internal.h"
#include "sv_q2.h"
#include "sv_stage.h"

namespace sv {

constexpr int LDS_BUDGET = 80 * 1024 - 256;   // two 512-thread blocks per CU (160 KB LDS)

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
  w.h = (float*)take(plain ? 0 : sizeof(float) * (size_t)max_assign * d->inter);
  w.hmax = (uint32_t*)take(sizeof(uint32_t) * max_assign);
  w.part = (float*)take(plain ? 0 : sizeof(float) * (size_t)max_assign * d->hidden);
  // column groups of at least one column: at most one item per unit plus one
  // per further column
  const int max_work = max_units + max_assign;
  w.work_gu = (MoeWork*)take(sizeof(MoeWork) * max_work);
  w.work_dn = (MoeWork*)take(sizeof(MoeWork) * max_work);
  void* xb = take(ximg_bytes(R, d->hidden, XL_PERM));
  if (p) w.x_img = ximg_carve(xb, R, d->hidden, XL_PERM);
  w.max_units = max_units;
  w.max_assign = max_assign;
  w.max_work = max_work;
  if (out) *out = w;
  return off;
}

// Activation rows are copied into LDS in 1 KB pieces.

__host__ __device__ inline int xl_pieces_per_row(int K, bool use_lo) {
  return ((2 * K + 1023) / 1024) * (use_lo ? 2 : 1) + (K / 4 + 1023) / 1024;
}

// Largest column group (rows per block) whose LDS copy fits the budget.
static int col_group(int K, bool use_lo, int R) {
  int cg = XL_MAX_COLS;
  while (cg > 1 && xl_bytes(cg, K, use_lo) > (size_t)LDS_BUDGET) --cg;
  return cg < R ? cg : R;
}

constexpr int DN_THREADS = 512;   // down: 8 waves, one 16-row tile each, all of inter
constexpr int DN_PAIRS = 4;       // staged (h row, 256-block) pairs per half-wave, at most
constexpr int DN_MAX_ROWS = 4;    // rows of a down descriptor: one int8 tile of 4 digit columns each

struct GpCfg;
static GpCfg gp_config(int hidden, int inter, bool use_lo, int R);

static int gateup_cols(const sv_moe_desc* d, int R, bool use_lo);

static int down_cols(const sv_moe_desc* d, int R) {
  int cg = DN_MAX_ROWS;
  while (cg > 1 && xl8_bytes(cg, d->inter) > (size_t)LDS_BUDGET) --cg;
  cg = cg < R ? cg : R;
  const int pair_cap = DN_PAIRS * (DN_THREADS / 32) / (d->inter / 256);
  if (cg > pair_cap) cg = pair_cap > 0 ? pair_cap : 1;
  return cg;
}

// ---------------------------------------------------- wave reductions (DPP)
// Reductions to lane 63 on the row-shift / row-broadcast network, then one
// readlane: a few cycles per step instead of an LDS round trip per shuffle.
template <int CTRL, int ROWS>
__device__ inline uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, ROWS, 0xF, false);
}

__device__ inline uint32_t wave_umax(uint32_t v) {
  v = max(v, dpp_u32<0x111, 0xF>(v));   // row_shr:1
  v = max(v, dpp_u32<0x112, 0xF>(v));   // row_shr:2
  v = max(v, dpp_u32<0x114, 0xF>(v));   // row_shr:4
  v = max(v, dpp_u32<0x118, 0xF>(v));   // row_shr:8   lane 15 of each row: the row's max
  v = max(v, dpp_u32<0x142, 0xA>(v));   // row_bcast:15 into rows 1 and 3
  v = max(v, dpp_u32<0x143, 0xC>(v));   // row_bcast:31 into rows 2 and 3
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
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

// Raises hmax[a] to |v| (bits; non-negative floats order as unsigned) with the
// largest value over the lane's 16-lane row: every lane of the row calls it
// (v = 0 where it has no value), lane 0 of the row does the atomic.
__device__ inline void note_hmax(uint32_t* hmax, int a, float v, bool any) {
  uint32_t m = __float_as_uint(fabsf(v));
  m = max(m, xlane<0xB1>(m));
  m = max(m, xlane<0x4E>(m));
  m = max(m, xlane<0x141>(m));
  m = max(m, xlane<0x140>(m));
  if (any && (__lane_id() & 15) == 0) atomicMax(hmax + a, m);
}

// ---------------------------------------------------------------- routing
constexpr int PREP_THREADS = 1024;

// One wave: top-k of one row of E logits (E <= 64 * PER), by logit, ties to
// the lower index; weights = softmax probability over all E.
template <int PER>
__device__ void route_row(const float* logits, int r, int E, int k, int* s_idx, int32_t* idx_out,
                          float* w_out, MoeWs ws) {
  const int lane = threadIdx.x & 63;
  uint32_t key[PER];
  float v[PER];
  unsigned taken = 0;
  uint32_t lk0 = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? logits[(size_t)r * E + e] : -INFINITY;
    key[i] = logit_key(v[i]);
    if (e >= E) taken |= 1u << i;
    else lk0 = max(lk0, key[i]);
  }
  const float mx = key_logit(wave_umax(lk0));   // the largest logit
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i)
    if (!(taken >> i & 1)) sum += expf(v[i] - mx);
  sum = wave_sum(sum);
  // k rounds of (largest key, then the lowest index holding it); lane s keeps
  // the s-th choice, and all k are written together afterwards
  uint32_t my_key = 0;
  int my_idx = 0;
  for (int s = 0; s < k; ++s) {
    uint32_t lk = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (!(taken >> i & 1)) lk = max(lk, key[i]);
    const uint32_t gk = wave_umax(lk);
    // the lowest index holding gk: the first slot i with a match, then the
    // lowest lane (index = lane + 64 i), from one ballot per slot
    int bi = -1;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const unsigned long long m = __ballot(!(taken >> i & 1) && key[i] == gk);
      if (bi < 0 && m) bi = 64 * i + (int)__builtin_ctzll(m);
    }
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (lane + 64 * i == bi) taken |= 1u << i;
    if (lane == s) {
      my_key = gk;
      my_idx = bi;
    }
  }
  if (lane < k) {
    const float w = expf(key_logit(my_key) - mx) / sum;
    s_idx[r * k + lane] = my_idx;
    ws.topk_idx[r * k + lane] = my_idx;
    ws.topk_w[r * k + lane] = w;
    if (idx_out) idx_out[r * k + lane] = my_idx;
    if (w_out) w_out[r * k + lane] = w;
  }
}

// Block 0 of the prep kernel: top-k of every row, then grouping.
// Work items of one expert kernel: each unit's assignments cut into groups
// of at most cg columns (wave 0).
__device__ void emit_work(const int* s_uexp, const int* s_uoff, const int* s_ucnt, int nu,
                          const int* s_arow, int cg, MoeWork* work, int* n_work) {
  const int lane = threadIdx.x & 63;
  int base = 0;
  for (int u0 = 0; u0 < nu; u0 += 64) {
    const int u = u0 + lane;
    const int ng = u < nu ? (s_ucnt[u] + cg - 1) / cg : 0;
    const int incl = wave_incl_scan(ng);
    for (int j = 0; j < ng; ++j) {
      MoeWork w;
      w.expert = s_uexp[u];
      w.a0 = s_uoff[u] + j * cg;
      w.ncols = min(cg, s_ucnt[u] - j * cg);
      w.pad = 0;
#pragma unroll
      for (int c = 0; c < MOE_WORK_COLS; ++c) w.rows[c] = c < w.ncols ? s_arow[w.a0 + c] : 0;
      work[base + incl - ng + j] = w;
    }
    base += __builtin_amdgcn_readlane(incl, 63);
  }
  if (lane == 0) *n_work = base;
}

__device__ void route_and_group(const float* logits, int R, int E, int k, int has_shared,
                                int cg_gu, int cg_dn, int32_t* idx_out, float* w_out, MoeWs ws) {
  __shared__ int s_idx[SV_MAX_ROWS * SV_MAX_TOPK];
  __shared__ unsigned long long s_rmask[SV_MAX_EXPERTS];   // rows that chose expert e (R <= 64)
  __shared__ int eoff[SV_MAX_EXPERTS];
  __shared__ int s_uexp[SV_MAX_EXPERTS + 1], s_uoff[SV_MAX_EXPERTS + 1], s_ucnt[SV_MAX_EXPERTS + 1];
  __shared__ int s_arow[SV_MAX_ROWS * (SV_MAX_TOPK + 1)];
  __shared__ int s_nu;
  const int tid = threadIdx.x, lane = tid & 63, wv = wave_id();
  constexpr int NW = PREP_THREADS / 64;
  for (int e = tid; e < E; e += PREP_THREADS) s_rmask[e] = 0ull;
  for (int a = tid; a < ws.max_assign; a += PREP_THREADS) ws.hmax[a] = 0u;   // gate/up raises them
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
  if (wv == 0) emit_work(s_uexp, s_uoff, s_ucnt, nu + has_shared, s_arow, cg_gu, ws.work_gu,
                         &ws.meta->n_work_gu);
  if (wv == 1) emit_work(s_uexp, s_uoff, s_ucnt, nu + has_shared, s_arow, cg_dn, ws.work_dn,
                         &ws.meta->n_work_dn);
}

template <int DT>
__global__ __launch_bounds__(PREP_THREADS) void k_moe_prep(const float* logits, int R, int E, int k,
                                                           int has_shared, int cg_gu, int cg_dn,
                                                           int32_t* idx_out, float* w_out,
                                                           const void* x, MoeWs ws) {
  __shared__ int sh[2 * PREP_THREADS / 64];
  if (blockIdx.x == 0) {
    route_and_group(logits, R, E, k, has_shared, cg_gu, cg_dn, idx_out, w_out, ws);
  } else {
    stage_row<DT, PREP_THREADS>(x, blockIdx.x - 1, XL_PERM, ws.x_img, sh);   // one block per row
  }
}

hipError_t launch_moe_prep(const sv_moe_desc* d, int R, const float* router_logits,
                           const void* x, int x_dtype, int32_t* topk_idx_out,
                           float* topk_w_out, MoeWs ws, hipStream_t s) {
  const int has_shared = d->s_gate ? 1 : 0;
  const dim3 grid(1 + R);
  const int cg_gu = gateup_cols(d, R, x_dtype == SV_F32), cg_dn = down_cols(d, R);
  if (x_dtype == SV_BF16)
    hipLaunchKernelGGL(k_moe_prep<SV_BF16>, grid, dim3(PREP_THREADS), 0, s, router_logits, R,
                       d->n_experts, d->top_k, has_shared, cg_gu, cg_dn, topk_idx_out, topk_w_out,
                       x, ws);
  else
    hipLaunchKernelGGL(k_moe_prep<SV_F32>, grid, dim3(PREP_THREADS), 0, s, router_logits, R,
                       d->n_experts, d->top_k, has_shared, cg_gu, cg_dn, topk_idx_out, topk_w_out,
                       x, ws);
  return hipGetLastError();
}

// ------------------------------------------------------------ LDS staging
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

// ------------------------------------------------------------- gate / up
struct ExpertPtrs {
  const uint8_t *g, *u, *dn;     // routed, expert-major
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
  P.bytes_gu = q2_bytes(d->inter, d->hidden);
  P.bytes_d = q2_bytes(d->hidden, d->inter);
  return P;
}

constexpr int GU_THREADS = 512;   // 8 waves: (gate, up) x 4 K-quarters of one 16-row tile

template <bool USE_LO, bool WIDE_D>
__global__ __launch_bounds__(GU_THREADS, 4) void k_q2_gateup(ExpertPtrs P, int hidden, int inter,
                                                             MoeWs ws) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int tile = blockIdx.x;
  const int nwork = ws.meta->n_work_gu;
  const MoeWork wk = ws.work_gu[blockIdx.y];   // in bounds for every launched block
  if ((int)blockIdx.y >= nwork) return;
  const int e = wk.expert, a0 = wk.a0, ncols = wk.ncols;
  const int* rows = ws.work_gu[blockIdx.y].rows;   // activation rows of the block's columns
  const int tid = threadIdx.x, lane = tid & 63, wv = wave_id();
  const int m = wv >> 2, q = wv & 3;
  const int nl = lane & 15, g = lane >> 4;
  const int n = tile * 16 + nl;
  const int nb = hidden / 256;
  const uint8_t* base = m == 0 ? (e >= 0 ? P.g + (size_t)e * P.bytes_gu : P.sg)
                               : (e >= 0 ? P.u + (size_t)e * P.bytes_gu : P.su);
  const Q2View W = q2_view(base, inter, hidden);
  const XLw L = xl_make(lds, ncols, hidden, USE_LO);
  f4_t acc = {0.f, 0.f, 0.f, 0.f};
  auto issue = [&]() { xl_img_dma(ws.x_img, rows, 0, ncols, USE_LO, L); };
  auto sync = [&](int nload) {
    wait_vmcnt_le(nload);   // this wave's copies (older than its nload weight loads) have landed
    barrier_keep_loads();
  };
  q2_range_staged<WIDE_D, USE_LO>(W, n, nb * q / 4, nb * (q + 1) / 4, xl_view(L), min(nl, ncols - 1),
                                  lane, acc, issue, sync);
  __syncthreads();   // every wave is done with the rows: reuse LDS for the partial sums
  f4_t* red = (f4_t*)lds;
  red[wv * 64 + lane] = acc;
  __syncthreads();
  if (wv != 0) return;
  const f4_t gs = ((red[lane] + red[64 + lane]) + red[128 + lane]) + red[192 + lane];
  const f4_t us = ((red[256 + lane] + red[320 + lane]) + red[384 + lane]) + red[448 + lane];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = 4 * g + i;   // (uniform in the lane's 16-lane row)
    float hv = 0.f;
    if (c < ncols) {
      const float rs = ws.x_img.rscale[rows[c]];
      const float gv = gs[i] * rs, uv = us[i] * rs;
      hv = gv / (1.f + expf(-gv)) * uv;
      ws.h[(size_t)(a0 + c) * inter + n] = hv;
    }
    note_hmax(ws.hmax, a0 + c, hv, c < ncols);
  }
}

// ------------------------------------------------ gate / up, persistent
// Blocks of 8 waves: wave (m, q) = (matrix gate/up, K part q of 4), each part
// NQ = nb / 4 consecutive 256-element blocks.  Block b owns the contiguous
// item range [b I / G, (b + 1) I / G) of the I = n_work * (inter/16) items
// (work descriptor, 16-row tile), which are ordered by descriptor, and every
// wave works on its (m, q) share of each item in turn.  A wave issues the
// next item's loads while it computes the current item -- the loads of the
// first half of its part once that half is computed, the rest after the
// second half -- so its loads stay in flight across items and across the
// per-item barrier.  The activation rows are copied into LDS only when the
// descriptor changes.  Partial sums meet in a double-buffered LDS area;
// wave (item mod 8) adds them up and applies SwiGLU.  Two blocks share a CU
// (four waves per SIMD, two of each block).
constexpr int GP_WAVES = 8, GP_PARTS = 4;
constexpr int GP_ZERO_BYTES = 8 * 512 + 64;   // zero operands of q2_block_c1: NQ <= 8 blocks

struct GpCfg {
  bool ok;
  int nq, cols;
  size_t lds;
};

// d/dmin window of a part starting at block kb0: 2 DW values from the even
// block w0 = kb0 & ~1 (even lane-rows d, odd lane-rows dmin, one dword per 2
// blocks); the part's values start at half (kb0 & 1) of it.
__host__ __device__ constexpr int gp_dw(int nq) { return (nq + (nq & 1) + 1) / 2; }

static GpCfg gp_config(int hidden, int inter, bool use_lo, int R) {
  GpCfg c{};
  const int nb = hidden / 256;
  if (hidden % 256 != 0 || nb % GP_PARTS != 0) return c;
  if ((size_t)inter * nb * 64 >= ((size_t)1 << 31)) return c;   // 32-bit load offsets (gp_load)
  c.nq = nb / GP_PARTS;
  if (c.nq < 1 || c.nq > 8) return c;
  const int dw = gp_dw(c.nq);
  if (dw > 4) return c;
  for (int q = 0; q < GP_PARTS; ++q)   // every window inside the row
    if ((c.nq * q & ~1) + 2 * dw > nb) return c;
  const size_t budget = (size_t)80 * 1024 - 512;   // two blocks per CU
  const size_t red = (size_t)2 * GP_WAVES * 64 * 16 + 2 * XL_MAX_COLS * 4 + GP_ZERO_BYTES;
  int cg = XL_MAX_COLS;
  while (cg > 1 && xl_bytes(cg, hidden, use_lo) + red > budget) --cg;
  if (xl_bytes(cg, hidden, use_lo) + red > budget) return c;
  c.cols = cg < R ? cg : R;
  c.lds = xl_bytes(c.cols, hidden, use_lo) + red;
  c.ok = true;
  return c;
}

// The loads of one half of a part: N code blocks, plus (first half) the
// block scales and the scale nibbles of the first 4 blocks, or (second half
// of a part of more than 4 blocks) the nibbles of blocks 4..7.  Nibble loads:
// lane-row g gets block base + g (clamped to the row).
template <int NQ, bool FIRST>
struct GpHalf {
  static constexpr int N0 = NQ > 4 ? 4 : (NQ + 1) / 2;
  static constexpr int N = FIRST ? N0 : NQ - N0;
  static constexpr bool SC = FIRST || NQ > 4;
  static constexpr int DW = FIRST ? gp_dw(NQ) : 0;
  static constexpr int LOADS = N + (SC ? 1 : 0) + (DW > 0 ? 1 : 0);
  uint4 qs[N > 0 ? N : 1];
  uint4 sc;
  uint32_t dd[DW > 0 ? DW : 1];
};

// (32-bit offsets from the planes' uniform bases: the loads take a scalar
// base and one offset register; the host keeps every plane under 2^31 bytes
// for the kernels that use this)
template <int NQ, bool FIRST>
__device__ __forceinline__ void gp_load(const Q2View& W, size_t rb, int kb0, int g,
                                        GpHalf<NQ, FIRST>& h) {
  using H = GpHalf<NQ, FIRST>;
  const uint32_t r0 = (uint32_t)rb;
  const int b0 = kb0 + (FIRST ? 0 : H::N0);
  if (H::SC) h.sc = *(const uint4*)(W.sc + (r0 + (uint32_t)min(b0 + g, W.nb - 1)) * 16u);
  if (H::DW > 0) {
    const uint16_t* dp = ((g & 1) ? W.dm : W.d) + (r0 + (uint32_t)(kb0 & ~1));
    if (H::DW == 1) {
      h.dd[0] = *(const uint32_t*)dp;
    } else if (H::DW == 2) {
      const uint2 v = *(const uint2*)dp;
      h.dd[0] = v.x;
      h.dd[1] = v.y;
    } else if (H::DW == 3) {
      const uint3 v = *(const uint3*)dp;
      h.dd[0] = v.x;
      h.dd[1] = v.y;
      h.dd[2] = v.z;
    } else {
      const uint4 v = *(const uint4*)dp;
      h.dd[0] = v.x;
      h.dd[1] = v.y;
      h.dd[2] = v.z;
      h.dd[3] = v.w;
    }
  }
  const uint8_t* q = W.qs + ((r0 + (uint32_t)b0) * 64u + 16u * (uint32_t)g);
#pragma unroll
  for (int i = 0; i < H::N; ++i) h.qs[i] = *(const uint4*)(q + 64 * i);
}

template <bool USE_LO, int NQ>
__global__ __launch_bounds__(GP_WAVES * 64, 4) void k_q2_gateup_p(ExpertPtrs P, int hidden, int inter,
                                                                  int CG, MoeWs ws) {
  extern __shared__ __align__(16) uint8_t lds[];
  using H0 = GpHalf<NQ, true>;
  using H1 = GpHalf<NQ, false>;
  constexpr int N0 = H0::N0, DW = H0::DW;
  const int T = inter / 16;
  const long total = (long)ws.meta->n_work_gu * T;
  // (the 64-bit divisions run on the vector unit: make the results uniform so
  // that descriptor reads are scalar loads)
  const int i0 = __builtin_amdgcn_readfirstlane((int)(total * blockIdx.x / gridDim.x));
  const int i1 = __builtin_amdgcn_readfirstlane((int)(total * (blockIdx.x + 1) / gridDim.x));
  if (i0 >= i1) return;
  const int lane = threadIdx.x & 63, wv = wave_id();
  const int m = wv >= GP_PARTS, q = wv & (GP_PARTS - 1);
  const int nl = lane & 15, g = lane >> 4;
  const int nb = hidden / 256, kb0 = NQ * q;
  const uint32_t dshift = 16 * (kb0 & 1);   // the part's first value: half (kb0 & 1) of the window
  const auto work = const_ptr(ws.work_gu);   // descriptor reads as scalar loads
  f4_t* red = (f4_t*)(lds + xl_bytes(CG, hidden, USE_LO));
  // row scales of a descriptor's columns, in LDS slot (descriptor index & 1):
  // the epilogue of the old descriptor's last item may still read its slot
  // while the next descriptor's scales are written
  float* rsc_slots = (float*)(lds + xl_bytes(CG, hidden, USE_LO) + (size_t)2 * GP_WAVES * 64 * 16);
  // zeros read by the idle lanes of single-row operands (q2_block_c1): one
  // part's worth of blocks, written once
  _Float16* zeros = (_Float16*)(rsc_slots + 2 * XL_MAX_COLS);
  for (int z = threadIdx.x; z < GP_ZERO_BYTES / 16; z += blockDim.x) ((uint4*)zeros)[z] = make_uint4(0, 0, 0, 0);
  auto wview = [&](int e) {
    const uint8_t* base = m == 0 ? (e >= 0 ? P.g + (size_t)e * P.bytes_gu : P.sg)
                                 : (e >= 0 ? P.u + (size_t)e * P.bytes_gu : P.su);
    return q2_view(base, inter, hidden);
  };

  // load cursor: the item whose weights are issued next (stays on the last
  // item of the range once there: those loads re-read cached lines and keep
  // the compiler's load counting identical on every path)
  int lw = __builtin_amdgcn_readfirstlane(i0 / T), lt = i0 - lw * T, li = i0;
  Q2View LW = wview(work[lw].expert);
  auto issue0 = [&](H0& h) { gp_load<NQ, true>(LW, (size_t)(lt * 16 + nl) * nb, kb0, g, h); };
  auto issue1 = [&](H1& h) {
    gp_load<NQ, false>(LW, (size_t)(lt * 16 + nl) * nb, kb0, g, h);
    if (li + 1 < i1) {
      ++li;
      if (++lt == T) {
        lt = 0;
        ++lw;
        LW = wview(work[lw].expert);
      }
    }
  };

  // compute cursor
  int w = lw, t = lt;
  int a0_cur = work[w].a0, nc_cur = work[w].ncols;
  auto row_scales = [&]() {
    if (wv == 0 && lane < XL_MAX_COLS)
      rsc_slots[(w & 1) * XL_MAX_COLS + lane] = lane < nc_cur ? ws.x_img.rscale[work[w].rows[lane]] : 0.f;
  };
  row_scales();
  // the first descriptor's activation copies, then the first item's weights
  xl_img_dma(ws.x_img, (const int*)work[w].rows, 0, nc_cur, USE_LO, xl_make(lds, nc_cur, hidden, USE_LO));
  H0 h0;
  H1 h1;
  issue0(h0);
  issue1(h1);
  wait_vmcnt_le(H0::LOADS + H1::LOADS);   // this wave's activation copies are done
  barrier_lds();

  for (int i = i0; i < i1; ++i) {
    const XLw L = xl_make(lds, nc_cur, hidden, USE_LO);   // rebuilt, not carried
    const int cr = min(nl, nc_cur - 1);
    const _Float16* xh = L.hi + (size_t)cr * L.rs + kb0 * 256 + g * 8;
    const _Float16* xl = L.lo + (size_t)cr * L.rs + kb0 * 256 + g * 8;
    const _Float16* xs = L.sx + (size_t)cr * L.sxs + kb0 * 32 + g * 8;
    f4_t acc = {0.f, 0.f, 0.f, 0.f};
    // block scales: both halves of the window to every lane, aligned so that
    // value b belongs to block kb0 + b
    uint32_t dv[DW], mv[DW];
#pragma unroll
    for (int j = 0; j < DW; ++j) {
      const auto sw = __builtin_amdgcn_permlane16_swap(h0.dd[j], h0.dd[j], false, false);
      dv[j] = sw[0];
      mv[j] = sw[1];
    }
#pragma unroll
    for (int j = 0; j < DW; ++j) {
      dv[j] = __builtin_amdgcn_alignbit(j + 1 < DW ? dv[j + 1] : 0u, dv[j], dshift);
      mv[j] = __builtin_amdgcn_alignbit(j + 1 < DW ? mv[j + 1] : 0u, mv[j], dshift);
    }
    // one activation row: sub-block selector operands (q2_block_c1); lane
    // (c, g) is live for the steps of sub-block c == 4g + u.  The branch is
    // uniform; both halves' loads are issued outside it.
    const bool one = nc_cur == 1;
    float ac = 0.f;
    auto sel = [&](uint32_t* ph, uint32_t* pl) {   // byte offsets from lds
      const uint32_t oh = (uint32_t)((const uint8_t*)xh - lds), ol = (uint32_t)((const uint8_t*)xl - lds);
      const uint32_t oz = (uint32_t)((const uint8_t*)zeros - lds);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool live = nl == 4 * g + u;
        ph[u] = live ? oh : oz - 128 * u;
        pl[u] = live ? ol : oz - 128 * u;
      }
    };
    {
      uint32_t sct[4];
      xpose4(h0.sc, sct);
      if (one) {
        uint32_t ph[4], pl[4];
        sel(ph, pl);
#pragma unroll
        for (int b = 0; b < NQ && b < 8; ++b) {
          if (b >= N0 && NQ > 4) break;
          // (second-half blocks of a part of at most 4 use the first nibble load)
          const uint4& qs = b < N0 ? h0.qs[b] : h1.qs[b - N0 < H1::N ? b - N0 : 0];
          q2_block_c1<USE_LO>(qs, sct[b & 3], win_val(dv, b), win_val(mv, b), g == 0, lds, ph, pl, 256 * b,
                              xs + 32 * b, ac);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
#pragma unroll
        for (int b = 0; b < NQ && b < 8; ++b) {
          if (b >= N0 && NQ > 4) break;
          const uint4& qs = b < N0 ? h0.qs[b] : h1.qs[b - N0 < H1::N ? b - N0 : 0];
          q2_block<USE_LO>(qs, sct[b & 3], win_val(dv, b), win_val(mv, b), xh + 256 * b, xl + 256 * b,
                           xs + 32 * b, acc);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    issue0(h0);
    if (NQ > 4) {
      uint32_t sct[4];
      xpose4(h1.sc, sct);
      if (one) {
        uint32_t ph[4], pl[4];
        sel(ph, pl);
#pragma unroll
        for (int b = N0; b < NQ; ++b) {
          q2_block_c1<USE_LO>(h1.qs[b - N0], sct[b - N0], win_val(dv, b), win_val(mv, b), g == 0, lds, ph, pl,
                              256 * b, xs + 32 * b, ac);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
#pragma unroll
        for (int b = N0; b < NQ; ++b) {
          q2_block<USE_LO>(h1.qs[b - N0], sct[b - N0], win_val(dv, b), win_val(mv, b), xh + 256 * b,
                           xl + 256 * b, xs + 32 * b, acc);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    issue1(h1);
    if (one) {
      // the row's total over its 4 lanes (g = 0..3), as column 0 of lane-row 0
      ac = rows_sum(ac);
      acc[0] = g == 0 ? ac : 0.f;
    }
    // partial sums of item i meet in buffer i & 1
    f4_t* rbuf = red + (size_t)(i & 1) * GP_WAVES * 64;
    rbuf[wv * 64 + lane] = acc;
    barrier_lds();
    if (wv == (i & (GP_WAVES - 1))) {
      // (addressed from the lane id, which the compiler recomputes instead of
      // keeping a register live across the item)
      const f4_t* rl = red + (size_t)(i & 1) * GP_WAVES * 64 + __lane_id();
      const f4_t gs = ((rl[0] + rl[64]) + rl[128]) + rl[192];
      const f4_t us = ((rl[256] + rl[320]) + rl[384]) + rl[448];
      const int n = t * 16 + nl;
      // (lane groups g >= 2 hold columns 8..15, never present: kept in bounds)
      const float* rsv = rsc_slots + (w & 1) * XL_MAX_COLS + min(4 * g, XL_MAX_COLS - 4);
      const int ne = min(4, nc_cur - 4 * g);   // (uniform in the lane's 16-lane row)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float hv = 0.f;
        if (e < ne) {
          const float gv = gs[e] * rsv[e], uv = us[e] * rsv[e];
          hv = gv / (1.f + __expf(-gv)) * uv;
          ws.h[(size_t)(a0_cur + 4 * g + e) * inter + n] = hv;
        }
        note_hmax(ws.hmax, a0_cur + 4 * g + e, hv, e < ne);
      }
    }
    // next compute item; a new descriptor's rows replace the old ones once
    // every wave is past item i
    if (++t == T && i + 1 < i1) {
      t = 0;
      ++w;
      a0_cur = work[w].a0;
      nc_cur = work[w].ncols;
      xl_img_dma(ws.x_img, (const int*)work[w].rows, 0, nc_cur, USE_LO, xl_make(lds, nc_cur, hidden, USE_LO));
      row_scales();
      wait_vmcnt_le(0);
      barrier_lds();
    }
  }
}

static size_t gu_lds(int hidden, bool use_lo, int CG) {
  const size_t x = xl_bytes(CG, hidden, use_lo), red = (size_t)GU_THREADS * 16;
  return x > red ? x : red;
}

static int gateup_cols(const sv_moe_desc* d, int R, bool use_lo) {
  const GpCfg c = gp_config(d->hidden, d->inter, use_lo, R);
  return c.ok ? c.cols : col_group(d->hidden, use_lo, R);
}

hipError_t launch_q2_gateup(const sv_moe_desc* d, int R, bool use_lo, MoeWs ws, hipStream_t s) {
  const ExpertPtrs P = expert_ptrs(d);
  const GpCfg c = gp_config(d->hidden, d->inter, use_lo, R);
  if (c.ok) {
    const dim3 grid(2 * cu_count()), block(64 * GP_WAVES);
#define SV_GP(Q)                                                                                   \
  case Q:                                                                                          \
    if (use_lo)                                                                                    \
      hipLaunchKernelGGL((k_q2_gateup_p<true, Q>), grid, block, c.lds, s, P, d->hidden, d->inter,  \
                         c.cols, ws);                                                              \
    else                                                                                           \
      hipLaunchKernelGGL((k_q2_gateup_p<false, Q>), grid, block, c.lds, s, P, d->hidden, d->inter, \
                         c.cols, ws);                                                              \
    break;
    switch (c.nq) { SV_GP(1) SV_GP(2) SV_GP(3) SV_GP(4) SV_GP(5) SV_GP(6) SV_GP(7) SV_GP(8) default: break; }
#undef SV_GP
    return hipGetLastError();
  }
  const int CG = gateup_cols(d, R, use_lo);
  const dim3 grid(d->inter / 16, ws.max_work, 1);
  const size_t lb = gu_lds(d->hidden, use_lo, CG);
  const bool wide = q2_wide_d(d->hidden / 256);
#define SV_GU(LO, WD)                                                                              \
  hipLaunchKernelGGL((k_q2_gateup<LO, WD>), grid, dim3(GU_THREADS), lb, s, P, d->hidden, d->inter, \
                     ws)
  if (use_lo) {
    if (wide) SV_GU(true, true); else SV_GU(true, false);
  } else {
    if (wide) SV_GU(false, true); else SV_GU(false, false);
  }
#undef SV_GU
  return hipGetLastError();
}

// ------------------------------------------------------------------ down

// h rows of a down descriptor into the int8 image (sv_q2.h, int8 form):
// half-wave hw converts the (row, 256-block) pairs hw, hw + 16, ... (at most
// PAIRS); lane l of a pair takes sub-block l/2, element positions j = 2(l&1)
// and 2(l&1) + 1, at b = 0..3 (elements 16 sb + 4b + j), so that it writes
// whole dwords of each digit plane.  The row's scale comes from its largest
// |h|, which the gate/up kernel left in hmax (loaded with the values).
template <int PAIRS>
struct DnH8 {
  float2 v[PAIRS][4];
  uint32_t m[DN_MAX_ROWS];   // hmax bits of the descriptor's rows (uniform: scalar registers)
};

template <int PAIRS>
__device__ __forceinline__ void dn8_h_load(const float* h, const uint32_t* hmax, int a0, int ncols, int inter,
                                           DnH8<PAIRS>& v) {
  const auto hm = const_ptr(hmax + a0);
#pragma unroll
  for (int j = 0; j < DN_MAX_ROWS; ++j) v.m[j] = hm[min(j, ncols - 1)];
  const int tid = threadIdx.x, l = tid & 31, hw = tid >> 5;
  const int sb = l >> 1, jh = l & 1;
  const int nbk = inter / 256, npairs = ncols * nbk;
#pragma unroll
  for (int i = 0; i < PAIRS; ++i) {
    const int p = hw + (DN_THREADS / 32) * i;
    if (p < npairs) {
      const int c = p / nbk, kb = p - c * nbk;
      const float* src = h + (size_t)(a0 + c) * inter + kb * 256 + 16 * sb + 2 * jh;
#pragma unroll
      for (int b = 0; b < 4; ++b) v.v[i][b] = *(const float2*)(src + 4 * b);
    }
  }
}

// Signed byte with the low 8 bits of x (sign-extended).
__device__ __forceinline__ int sbyte(int x) { return (x << 24) >> 24; }

template <int PAIRS>
__device__ __forceinline__ void dn8_h_convert(const DnH8<PAIRS>& v, int8_t* q, _Float16* sx, float* csc, int ncols,
                                              int inter) {
  const int tid = threadIdx.x, l = tid & 31, hw = tid >> 5;
  const int sb = l >> 1, jh = l & 1;
  const int nbk = inter / 256, npairs = ncols * nbk;
  const int rs = inter + 16, sxs = inter / 16;
#pragma unroll
  for (int i = 0; i < PAIRS; ++i) {   // digits
    const int p = hw + (DN_THREADS / 32) * i;
    if (p < npairs) {
      const int c = p / nbk, kb = p - c * nbk;
      const uint32_t mb = c == 0 ? v.m[0] : c == 1 ? v.m[1] : c == 2 ? v.m[2] : v.m[3];
      const float mx = __uint_as_float(mb);
      const int bad = mb >= 0x7F800000u;   // an infinite or NaN value in the row
      // |h| 2^e < 2^29: the leading digit stays within +-65
      int e = 0;
      if (mx > 0.f && !bad) {
        int E;
        frexpf(mx, &E);   // mx in [2^(E-1), 2^E)
        e = min(max(29 - E, -120), 120);
      }
      uint32_t w[4][2];   // [digit][j - 2 jh]
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
#pragma unroll
        for (int d = 0; d < 4; ++d) w[d][jj] = 0u;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const float x = jj == 0 ? v.v[i][b].x : v.v[i][b].y;
          const int a = bad ? 0 : (int)rintf(ldexpf(x, e));
          const int p3 = sbyte(a), a1 = (a - p3) >> 8;
          const int p2 = sbyte(a1), a2 = (a1 - p2) >> 8;
          const int p1 = sbyte(a2), p0 = (a2 - p1) >> 8;
          const int dg[4] = {p0, p1, p2, p3};
#pragma unroll
          for (int d = 0; d < 4; ++d) w[d][jj] |= ((uint32_t)dg[d] & 0xFFu) << (8 * b);
        }
      }
      // digit sums of the lane's 8 elements: the signed bytes of its two words
      int ps[4];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const int s1 = __builtin_amdgcn_sdot4((int)w[d][1], 0x01010101, 0, false);
        ps[d] = __builtin_amdgcn_sdot4((int)w[d][0], 0x01010101, s1, false);
      }
      // plane byte kb*256 + 64 t + 16 g + 4 j + b for sub-block sb = 4 g + t
      const int off = kb * 256 + 64 * (sb & 3) + 16 * (sb >> 2) + 8 * jh;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        *(uint2*)(q + (size_t)(4 * c + d) * rs + off) = make_uint2(w[d][0], w[d][1]);
        const int tot = ps[d] + (int)xlane<0xB1>((uint32_t)ps[d]);   // the partner lane's j
        if (jh == 0) sx[(size_t)(4 * c + d) * sxs + kb * 16 + sb] = (_Float16)(float)tot;
      }
      if (kb == 0 && l < 4)
        csc[4 * c + l] = bad ? __builtin_nanf("") : ldexpf(1.f, 24 - 8 * l - e);
    }
  }
  for (int c = tid; c < 16; c += blockDim.x)
    if (c >= 4 * ncols) csc[c] = 0.f;
  barrier_lds();   // (LDS only: the weight loads in flight are not waited for)
}

// Down projection on the int8 matrix cores: one block per (128-row group of
// hidden, descriptor of at most 4 rows), 8 waves of one 16-row tile over all
// of inter; the block's h rows are read into registers before the weight
// loads and converted into the LDS image (fixed-point digits, sv_q2.h).
template <bool WIDE_D, int PAIRS>
__global__ __launch_bounds__(DN_THREADS, 4) void k_q2_down(ExpertPtrs P, int hidden, int inter, MoeWs ws) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int nwork = ws.meta->n_work_dn;
  const MoeWork wk = ws.work_dn[blockIdx.y];   // in bounds for every launched block
  if ((int)blockIdx.y >= nwork) return;
  const int e = wk.expert, a0 = wk.a0, ncols = wk.ncols;
  const int lane = threadIdx.x & 63, wv = wave_id();
  const int nl = lane & 15, g = lane >> 4;
  const int n = (blockIdx.x * 8 + wv) * 16 + nl;
  const Q2View D = q2_view(e >= 0 ? P.dn + (size_t)e * P.bytes_d : P.sd, hidden, inter);
  int8_t* q;
  _Float16* sx;
  float* csc;
  xl8_carve(lds, ncols, inter, q, sx, csc);
  XL8 X;
  X.q = q;
  X.sx = sx;
  X.csc = csc;
  X.rs = inter + 16;
  X.sxs = inter / 16;
  DnH8<PAIRS> hv;
  f4_t acc = {0.f, 0.f, 0.f, 0.f};
  q2_range_staged_i8<WIDE_D>(
      D, n, 0, inter / 256, X, ncols, lane, acc, [&]() { dn8_h_load(ws.h, ws.hmax, a0, ncols, inter, hv); },
      [&](int) { dn8_h_convert(hv, q, sx, csc, ncols, inter); });
  // lane (n, g) holds tile columns 4g..4g+3: the four digits of row g
  if (g < ncols) {
    const f4_t sc = *(const f4_t*)(csc + 4 * g);
    ws.part[(size_t)(a0 + g) * hidden + n] = ((sc[0] * acc[0] + sc[1] * acc[1]) + sc[2] * acc[2]) + sc[3] * acc[3];
  }
}

hipError_t launch_q2_down(const sv_moe_desc* d, int R, MoeWs ws, float* y, hipStream_t s) {
  const int CG = down_cols(d, R), nbk = d->inter / 256;
  const dim3 grid(d->hidden / 128, ws.max_work, 1);
  const ExpertPtrs P = expert_ptrs(d);
  const size_t lb = xl8_bytes(CG, d->inter);
  // staging registers for 2 (row, block) pairs per half-wave when that covers the rows
  const bool wide = q2_wide_d(nbk), few = CG * nbk <= 2 * (DN_THREADS / 32);
#define SV_DN(WD, PR) \
  hipLaunchKernelGGL((k_q2_down<WD, PR>), grid, dim3(DN_THREADS), lb, s, P, d->hidden, d->inter, ws)
  if (wide) {
    if (few) SV_DN(true, 2); else SV_DN(true, DN_PAIRS);
  } else {
    if (few) SV_DN(false, 2); else SV_DN(false, DN_PAIRS);
  }
#undef SV_DN
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_moe_combine(d, R, ws, y, s);
}

// --------------------------------------------------------------- combine
// y[r, n] = sum_{s<k} w[r, s] * part[a(r, s), n] (+ part[a(r, shared), n]), in slot order.
__global__ __launch_bounds__(256) void k_moe_combine(int hidden, int k, int has_shared, MoeWs ws,
                                                     float* y) {
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
    if (s < ns) v[s] = *(const float4*)(ws.part + (size_t)s_a[s] * hidden + 4 * n4);
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
  hipLaunchKernelGGL(k_moe_combine, dim3((d->hidden / 4 + 255) / 256, R), dim3(256), 0, s,
                     d->hidden, d->top_k, d->s_gate ? 1 : 0, ws, y);
  return hipGetLastError();
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

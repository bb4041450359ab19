// Routed two-bit MoE layer: routing + grouping, fused gate/up/SwiGLU, down
// projection with a fixed-order weighted combine, and the one-matrix form.
//
// Launch sequence of one layer (all on the caller's stream, no host sync):
//   k_moe_prep    block 0 routes all rows (top-k on logits, softmax weights)
//                 and groups (row, slot) pairs by expert so each touched
//                 expert's weights are read once ("MoE gate_up expert dedup",
//                 ds4-on-spark README, introduction); the other blocks stage x.
//   k_q2_gateup   grid (n-tile of inter, unit, column group): 4 waves split K,
//                 one pass computes gate and up and applies SwiGLU ("fused
//                 gate+up+swiglu MoE decode", 1x Spark tuned DSpark thread,
//                 Q&A answer 3).  h is kept in fp32.
//   k_stage       stages h per (row, slot) assignment.
//   k_q2_down     grid (64-row group of hidden, unit, column group); each wave
//                 one 16-row tile over all of inter; per-assignment outputs go
//                 to the workspace.
//   k_moe_combine y = fixed-order weighted sum of the per-assignment outputs:
//                 slots 0..k-1, then the shared expert.
// Blocks never wait on each other inside a kernel: on a part whose L2 is split
// across dies, a device-wide fence per block would cost far more than the
// extra launch.
#include "sv_internal.h"
#include "sv_q2.h"
#include "sv_stage.h"

namespace sv {

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
  w.part = (float*)take(plain ? 0 : sizeof(float) * (size_t)max_assign * d->hidden);
  void* xb = take(ximg_bytes(R, d->hidden, XL_PERM));
  void* hb = take(plain ? 0 : ximg_bytes(max_assign, d->inter, XL_PERM));
  if (p) {
    w.x_img = ximg_carve(xb, R, d->hidden, XL_PERM);
    if (!plain) w.h_img = ximg_carve(hb, max_assign, d->inter, XL_PERM);
  }
  w.max_units = max_units;
  w.max_assign = max_assign;
  if (out) *out = w;
  return off;
}

// ---------------------------------------------------------------- routing
__device__ inline bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

__device__ inline void wave_argmax(float& bv, int& bi) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float ov = __shfl_xor(bv, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    if (better(ov, oi, bv, bi)) {
      bv = ov;
      bi = oi;
    }
  }
}

__device__ inline float wave_max_f(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ inline float wave_sum_f(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Block 0: top-k + grouping.  256 threads.
__device__ void route_and_group(const float* logits, int R, int E, int k, int has_shared,
                                int32_t* idx_out, float* w_out, MoeWs ws) {
  __shared__ int s_idx[SV_MAX_ROWS * SV_MAX_TOPK];
  __shared__ int cnt[SV_MAX_EXPERTS];
  __shared__ int eoff[SV_MAX_EXPERTS];
  __shared__ int s_nu;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int e = tid; e < E; e += 256) cnt[e] = 0;
  if (logits == nullptr) {  // one expert, no router: weight 1
    for (int i = tid; i < R * k; i += 256) {
      s_idx[i] = 0;
      ws.topk_idx[i] = 0;
      ws.topk_w[i] = 1.f;
      if (idx_out) idx_out[i] = 0;
      if (w_out) w_out[i] = 1.f;
    }
  } else {
    constexpr int PER = SV_MAX_EXPERTS / 64;
    for (int r = wv; r < R; r += 4) {
      float v[PER];
      unsigned taken = 0;
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int e = lane + 64 * i;
        v[i] = e < E ? logits[(size_t)r * E + e] : -INFINITY;
        if (e >= E) taken |= 1u << i;
        mx = fmaxf(mx, v[i]);
      }
      mx = wave_max_f(mx);
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < PER; ++i)
        if (!(taken >> i & 1)) sum += expf(v[i] - mx);
      sum = wave_sum_f(sum);
      for (int s = 0; s < k; ++s) {
        float bv = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
          const int e = lane + 64 * i;
          if (!(taken >> i & 1) && better(v[i], e, bv, bi)) {
            bv = v[i];
            bi = e;
          }
        }
        wave_argmax(bv, bi);
        if (bi == 0x7fffffff) {  // only unordered (NaN) values left: lowest free index
          int fi = 0x7fffffff;
#pragma unroll
          for (int i = 0; i < PER; ++i)
            if (!(taken >> i & 1)) fi = min(fi, lane + 64 * i);
#pragma unroll
          for (int o = 32; o >= 1; o >>= 1) fi = min(fi, __shfl_xor(fi, o, 64));
          bi = fi;
        }
#pragma unroll
        for (int i = 0; i < PER; ++i)
          if (lane + 64 * i == bi) taken |= 1u << i;
        if (lane == 0) {
          const float w = expf(bv - mx) / sum;
          s_idx[r * k + s] = bi;
          ws.topk_idx[r * k + s] = bi;
          ws.topk_w[r * k + s] = w;
          if (idx_out) idx_out[r * k + s] = bi;
          if (w_out) w_out[r * k + s] = w;
        }
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < R * k; i += 256) atomicAdd(&cnt[s_idx[i]], 1);
  __syncthreads();
  if (wv == 0) {  // touched experts in ascending order -> units, assignment offsets
    int base_u = 0, base_a = 0;
    for (int c0 = 0; c0 < E; c0 += 64) {
      const int e = c0 + lane;
      const int ce = e < E ? cnt[e] : 0;
      int fu = ce > 0 ? 1 : 0, fa = ce;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int tu = __shfl_up(fu, o, 64), ta = __shfl_up(fa, o, 64);
        if (lane >= o) {
          fu += tu;
          fa += ta;
        }
      }
      const int u = base_u + fu - (ce > 0 ? 1 : 0);
      const int a = base_a + fa - ce;
      if (e < E) eoff[e] = a;
      if (ce > 0) {
        ws.unit_expert[u] = e;
        ws.unit_off[u] = a;
        ws.unit_cnt[u] = ce;
      }
      base_u += __shfl(fu, 63, 64);
      base_a += __shfl(fa, 63, 64);
    }
    if (lane == 0) s_nu = base_u;
  }
  __syncthreads();
  const int nu = s_nu;
  for (int i = tid; i < R * k; i += 256) {
    const int r = i / k, s = i - r * k, e = s_idx[i];
    int rank = 0;  // rows before r that chose e (each row picks an expert at most once)
    for (int j = 0; j < r * k; ++j) rank += s_idx[j] == e;
    const int a = eoff[e] + rank;
    ws.arow[a] = r;
    ws.amap[r * (k + 1) + s] = a;
  }
  if (has_shared) {
    for (int r = tid; r < R; r += 256) {
      ws.arow[R * k + r] = r;
      ws.amap[r * (k + 1) + k] = R * k + r;
    }
    if (tid == 0) {
      ws.unit_expert[nu] = -1;
      ws.unit_off[nu] = R * k;
      ws.unit_cnt[nu] = R;
    }
  }
  if (tid == 0) {
    ws.meta->n_units = nu + has_shared;
    ws.meta->n_assign = R * k + has_shared * R;
  }
}

template <int DT>
__global__ __launch_bounds__(256) void k_moe_prep(const float* logits, int R, int E, int k,
                                                  int has_shared, int32_t* idx_out, float* w_out,
                                                  const void* x, MoeWs ws) {
  if (blockIdx.x == 0) {
    route_and_group(logits, R, E, k, has_shared, idx_out, w_out, ws);
  } else {
    stage_gid<DT>(x, R, XL_PERM, ws.x_img, (blockIdx.x - 1) * 8 + (threadIdx.x >> 5),
                  threadIdx.x & 31);
  }
}

hipError_t launch_moe_prep(const sv_moe_desc* d, int R, const float* router_logits,
                           const void* x, int x_dtype, int32_t* topk_idx_out,
                           float* topk_w_out, MoeWs ws, hipStream_t s) {
  const int has_shared = d->s_gate ? 1 : 0;
  const int groups = R * (d->hidden / 256);
  const dim3 grid(1 + (groups + 7) / 8);
  if (x_dtype == SV_BF16)
    hipLaunchKernelGGL(k_moe_prep<SV_BF16>, grid, dim3(256), 0, s, router_logits, R, d->n_experts,
                       d->top_k, has_shared, topk_idx_out, topk_w_out, x, ws);
  else
    hipLaunchKernelGGL(k_moe_prep<SV_F32>, grid, dim3(256), 0, s, router_logits, R, d->n_experts,
                       d->top_k, has_shared, topk_idx_out, topk_w_out, x, ws);
  return hipGetLastError();
}

// ------------------------------------------------------------- gate / up
struct ExpertPtrs {
  const uint8_t *g, *u, *dn;     // routed, expert-major
  const uint8_t *sg, *su, *sd;   // shared
  size_t bytes_gu, bytes_d;
};

template <bool USE_LO>
__global__ __launch_bounds__(256) void k_q2_gateup(ExpertPtrs P, int hidden, int inter, MoeWs ws) {
  const int nt = blockIdx.x, u = blockIdx.y, cg = blockIdx.z;
  if (u >= ws.meta->n_units) return;
  const int e = ws.unit_expert[u], off = ws.unit_off[u], cnt = ws.unit_cnt[u];
  const int c0 = cg * 16;
  if (c0 >= cnt) return;
  Q2View W[2];
  W[0] = q2_view(e >= 0 ? P.g + (size_t)e * P.bytes_gu : P.sg, inter, hidden);
  W[1] = q2_view(e >= 0 ? P.u + (size_t)e * P.bytes_gu : P.su, inter, hidden);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int nl = lane & 15, g = lane >> 4;
  const int n = nt * 16 + nl;
  const XRow x = xrow(ws.x_img, (c0 + nl < cnt) ? ws.arow[off + c0 + nl] : -1, ws.arow[off]);
  const int nb = hidden / 256;
  const int kb0 = nb * wv / 4;
  f4_t acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  q2_run<2, USE_LO>(W, n, kb0, nb * (wv + 1) / 4 - kb0, x, lane, acc);
  __shared__ f4_t red[2][4][64];
  red[0][wv][lane] = acc[0];
  red[1][wv][lane] = acc[1];
  __syncthreads();
  if (wv != 0) return;
  f4_t sg = red[0][0][lane], su = red[1][0][lane];
#pragma unroll
  for (int w = 1; w < 4; ++w) {
    sg += red[0][w][lane];
    su += red[1][w][lane];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = c0 + 4 * g + i;
    if (c >= cnt) continue;
    const float gv = sg[i], uv = su[i];
    ws.h[(size_t)(off + c) * inter + n] = gv / (1.f + expf(-gv)) * uv;
  }
}

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

hipError_t launch_q2_gateup(const sv_moe_desc* d, int R, bool use_lo, MoeWs ws,
                            hipStream_t s) {
  const dim3 grid(d->inter / 16, ws.max_units, (R + 15) / 16);
  if (use_lo)
    hipLaunchKernelGGL(k_q2_gateup<true>, grid, dim3(256), 0, s, expert_ptrs(d), d->hidden,
                       d->inter, ws);
  else
    hipLaunchKernelGGL(k_q2_gateup<false>, grid, dim3(256), 0, s, expert_ptrs(d), d->hidden,
                       d->inter, ws);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // h -> image, one block per assignment actually present
  return launch_stage(ws.h, SV_F32, ws.max_assign, d->inter, XL_PERM, &ws.meta->n_assign,
                      ws.h_img, s);
}

// ------------------------------------------------------------------ down
// Grid (64-row group of hidden, unit, group of 4 columns).  The block's (up
// to 4) h rows are staged in LDS once -- all 4 waves use the same rows over
// all of inter -- then each wave streams one 16-row tile of the down matrix.
constexpr int DOWN_COLS = 4;

__host__ __device__ inline size_t down_lds_bytes(int inter) {
  return (size_t)DOWN_COLS * inter * 2 * 2 + (size_t)DOWN_COLS * (inter / 16) * 2 * 2 +
         (size_t)DOWN_COLS * (inter / 256) * 4;
}

__global__ __launch_bounds__(256) void k_q2_down(ExpertPtrs P, int hidden, int inter, MoeWs ws) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int grp = blockIdx.x, u = blockIdx.y, cg = blockIdx.z;
  if (u >= ws.meta->n_units) return;
  const int e = ws.unit_expert[u], off = ws.unit_off[u], cnt = ws.unit_cnt[u];
  const int c0 = cg * DOWN_COLS;
  if (c0 >= cnt) return;
  const int ncols = min(DOWN_COLS, cnt - c0);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nl = lane & 15;
  const int n = grp * 64 + wv * 16 + nl;
  const int nbk = inter / 256;
  XLds X;
  X.K = inter;
  X.nbk = nbk;
  _Float16* hi = (_Float16*)lds;
  _Float16* lo = hi + DOWN_COLS * inter;
  _Float16* sxh = lo + DOWN_COLS * inter;
  _Float16* sxl = sxh + DOWN_COLS * (inter / 16);
  float* bs = (float*)(sxl + DOWN_COLS * (inter / 16));
  X.hi = hi;
  X.lo = lo;
  X.sxh = sxh;
  X.sxl = sxl;
  X.bs = bs;
  // stage the rows of assignments off+c0 .. off+c0+ncols-1 (16-byte pieces)
  const XImg& H = ws.h_img;
  for (int c = 0; c < ncols; ++c) {
    const size_t a = (size_t)(off + c0 + c);
    for (int i = tid; i < inter / 8; i += 256) {
      *(uint4*)(hi + c * inter + 8 * i) = *(const uint4*)(H.hi + a * inter + 8 * i);
      *(uint4*)(lo + c * inter + 8 * i) = *(const uint4*)(H.lo + a * inter + 8 * i);
    }
    for (int i = tid; i < inter / 16; i += 256) {
      sxh[c * (inter / 16) + i] = H.sxh[a * (inter / 16) + i];
      sxl[c * (inter / 16) + i] = H.sxl[a * (inter / 16) + i];
    }
    for (int i = tid; i < nbk; i += 256) bs[c * nbk + i] = H.bscale[a * nbk + i];
  }
  __syncthreads();
  const Q2View D = q2_view(e >= 0 ? P.dn + (size_t)e * P.bytes_d : P.sd, hidden, inter);
  f4_t acc = {0.f, 0.f, 0.f, 0.f};
  // lane column c = nl reads LDS row nl & 3; columns >= ncols are padding (not stored)
  q2_run_lds(D, n, nbk, X, nl & 3, lane, acc);
  const int g = lane >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = 4 * g + i;   // tile column; only 0..ncols-1 are real
    if (c < ncols) ws.part[(size_t)(off + c0 + c) * hidden + n] = acc[i];
  }
}

hipError_t launch_q2_down(const sv_moe_desc* d, int R, MoeWs ws, float* y, hipStream_t s) {
  const dim3 grid(d->hidden / 64, ws.max_units, (R + DOWN_COLS - 1) / DOWN_COLS);
  hipLaunchKernelGGL(k_q2_down, grid, dim3(256), down_lds_bytes(d->inter), s, expert_ptrs(d),
                     d->hidden, d->inter, ws);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_moe_combine(d, R, ws, y, s);
}

// --------------------------------------------------------------- combine
// y[r, n] = sum_{s<k} w[r, s] * part[a(r, s), n] (+ part[a(r, shared), n]), in slot order.
// Grid (hidden/256, R): the row's slot map goes to LDS first, then all of its
// partial loads are issued together.
__global__ __launch_bounds__(256) void k_moe_combine(int hidden, int k, int has_shared, MoeWs ws,
                                                     float* y) {
  __shared__ int s_a[SV_MAX_TOPK + 1];
  __shared__ float s_w[SV_MAX_TOPK];
  const int r = blockIdx.y, tid = threadIdx.x;
  if (tid <= k) s_a[tid] = ws.amap[r * (k + 1) + tid];
  if (tid < k) s_w[tid] = ws.topk_w[r * k + tid];
  __syncthreads();
  const int n = blockIdx.x * 256 + tid;
  if (n >= hidden) return;
  const int ns = k + has_shared;
  float v[SV_MAX_TOPK + 1];
#pragma unroll
  for (int s = 0; s <= SV_MAX_TOPK; ++s)
    if (s < ns) v[s] = ws.part[(size_t)s_a[s] * hidden + n];
  float acc = 0.f;
#pragma unroll
  for (int s = 0; s < SV_MAX_TOPK; ++s)
    if (s < k) acc = fmaf(s_w[s], v[s], acc);
  if (has_shared) acc += v[k];
  y[(size_t)r * hidden + n] = acc;
}

hipError_t launch_moe_combine(const sv_moe_desc* d, int R, MoeWs ws, float* y, hipStream_t s) {
  hipLaunchKernelGGL(k_moe_combine, dim3((d->hidden + 255) / 256, R), dim3(256), 0, s, d->hidden,
                     d->top_k, d->s_gate ? 1 : 0, ws, y);
  return hipGetLastError();
}

// ----------------------------------------------------------------- plain
// y[R, n_out] = W x for one two-bit matrix; each wave one 16-row tile over all K.
template <bool USE_LO>
__global__ __launch_bounds__(256) void k_q2_plain(const uint8_t* w, int n_out, int k_in, int R,
                                                  XImg img, float* y) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int nt = blockIdx.x * 4 + wv, cg = blockIdx.z;
  if (nt * 16 >= n_out) return;
  const int nl = lane & 15, g = lane >> 4;
  const int n = nt * 16 + nl;
  const int nld = n < n_out ? n : n_out - 1;   // ragged tail: load a valid row, drop the result
  const Q2View W = q2_view(w, n_out, k_in);
  const int c = cg * 16 + nl;
  const XRow x = xrow(img, c < R ? c : -1, 0);
  f4_t acc = {0.f, 0.f, 0.f, 0.f};
  q2_run<1, USE_LO>(&W, nld, 0, W.nb, x, lane, &acc);
  if (n >= n_out) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int cc = cg * 16 + 4 * g + i;
    if (cc < R) y[(size_t)cc * n_out + n] = acc[i];
  }
}

hipError_t launch_q2_plain(const sv_moe_desc* d, int R, bool use_lo, MoeWs ws, float* y,
                           hipStream_t s) {
  const int tiles = (d->inter + 15) / 16;
  const dim3 grid((tiles + 3) / 4, 1, (R + 15) / 16);
  if (use_lo)
    hipLaunchKernelGGL(k_q2_plain<true>, grid, dim3(256), 0, s, (const uint8_t*)d->w_gate,
                       d->inter, d->hidden, R, ws.x_img, y);
  else
    hipLaunchKernelGGL(k_q2_plain<false>, grid, dim3(256), 0, s, (const uint8_t*)d->w_gate,
                       d->inter, d->hidden, R, ws.x_img, y);
  return hipGetLastError();
}

}  // namespace sv

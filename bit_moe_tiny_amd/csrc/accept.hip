// The p/q accept/reject rule with residual resampling, on the GPU.
//
// Rule (GB10/GX10 DSpark thread, post 1): drafts are sampled from q, the
// target defines p, a draft is accepted with probability min(1, p/q), a
// rejected draft is replaced from the normalised positive residual
// max(0, p - q); the verifier's K+1 rows give a bonus token when every draft
// passes.  Decided here with explicit uniforms: accept iff u_i q_i(d_i) <
// p_i(d_i), tested exactly as the sign of fma(u, q, -p); the replacement or
// bonus token is the first x whose running sum exceeds u_K times the total.
//
// Three launches, no host sync, no block waiting on another:
//   k_acc_stats  grid (chunk, row): per 2048-entry chunk of every target and
//                draft row, the chunk max of z/T and sum exp(z/T - max) in
//                fp64 (or the plain sum for probability rows), plus a
//                validity flag.  Spreads the vocabulary-wide reductions over
//                many CUs.
//   k_acc_chunk  grid (chunk, sequence): every block recombines its
//                sequence's row statistics (same order in every block, so all
//                agree bit for bit), replays the accept chain, and sums the
//                sampling weights of its chunk (residual, or p_K for the
//                bonus).
//   k_acc_pick   one block per sequence: prefix over the chunk totals, the
//                chunk that holds u_K * Z, a block scan inside it, outputs.
#include "sv_internal.h"

namespace sv {

constexpr int ACC_CHUNK = 2048;
constexpr int ACC_PER = ACC_CHUNK / 256;
constexpr int ACC_MAX_CH = 256;   // V <= 524288

struct AccWs {
  double* cmax;     // [rows, CH]
  double* csum;     // [rows, CH]
  int* cbad;        // [rows, CH]
  double* rsum;     // [S, CH]   sampling weight per chunk
  double* sst;      // [S, 4]    pm, pz, qm, qz of the sampled row pair
  int* sinfo;       // [S, 2]    n accepted, invalid
};

static inline int acc_chunks(int V) { return (V + ACC_CHUNK - 1) / ACC_CHUNK; }

static AccWs acc_carve(void* base, int S, int K, int V) {
  const size_t rows = (size_t)S * (2 * K + 1), CH = acc_chunks(V);
  uint8_t* p = (uint8_t*)base;
  AccWs w;
  w.cmax = (double*)p;
  p += up256(rows * CH * 8);
  w.csum = (double*)p;
  p += up256(rows * CH * 8);
  w.cbad = (int*)p;
  p += up256(rows * CH * 4);
  w.rsum = (double*)p;
  p += up256((size_t)S * CH * 8);
  w.sst = (double*)p;
  p += up256((size_t)S * 4 * 8);
  w.sinfo = (int*)p;
  return w;
}

size_t accept_ws_bytes(int S, int K, int V) {
  const size_t rows = (size_t)S * (2 * K + 1), CH = acc_chunks(V);
  return 2 * up256(rows * CH * 8) + up256(rows * CH * 4) + up256((size_t)S * CH * 8) +
         up256((size_t)S * 4 * 8) + up256((size_t)S * 2 * 4);
}

__device__ inline double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ inline double wave_max_d(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmax(v, __shfl_xor(v, o, 64));
  return v;
}

// Block-wide fixed-order reductions (256 threads); `sh` holds 4 doubles.
__device__ inline double block_sum_d(double v, double* sh) {
  v = wave_sum_d(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  return ((sh[0] + sh[1]) + sh[2]) + sh[3];
}
__device__ inline double block_max_d(double v, double* sh) {
  v = wave_max_d(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  return fmax(fmax(sh[0], sh[1]), fmax(sh[2], sh[3]));
}

// Block-wide exclusive prefix sum in a fixed order (256 threads); returns the
// exclusive prefix and sets *total.  `sh` holds 4 doubles.
__device__ inline double block_excl_scan_d(double v, double* sh, double* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  double inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double t = __shfl_up(inc, o, 64);
    if (lane >= o) inc += t;
  }
  __syncthreads();
  if (lane == 63) sh[wv] = inc;
  __syncthreads();
  double base = 0.0;
  for (int w = 0; w < wv; ++w) base += sh[w];
  *total = ((sh[0] + sh[1]) + sh[2]) + sh[3];
  return base + inc - v;
}

struct RowSrc {
  const float* p;   // row start
  int kind;         // SV_LOGITS / SV_PROBS
  double T;
};

__device__ inline RowSrc row_src(int r, int S, int K, int V, const float* target, int tkind,
                                 float Tp, const float* draft, int dkind, float Tq) {
  RowSrc s;
  const int nt = S * (K + 1);
  if (r < nt) {
    s.p = target + (size_t)r * V;
    s.kind = tkind;
    s.T = (double)Tp;
  } else {
    s.p = draft + (size_t)(r - nt) * V;
    s.kind = dkind;
    s.T = (double)Tq;
  }
  return s;
}

__global__ __launch_bounds__(256) void k_acc_stats(int S, int K, int V, const float* target,
                                                   int tkind, float Tp, const float* draft,
                                                   int dkind, float Tq, AccWs ws) {
  __shared__ double sh[4];
  __shared__ int shb[4];
  const int c = blockIdx.x, r = blockIdx.y, CH = gridDim.x;
  const RowSrc src = row_src(r, S, K, V, target, tkind, Tp, draft, dkind, Tq);
  const int x0 = c * ACC_CHUNK;
  double a[ACC_PER];
  int bad = 0;
  double mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < ACC_PER; ++i) {
    const int x = x0 + threadIdx.x + 256 * i;
    a[i] = -INFINITY;
    if (x < V) {
      const float v = src.p[x];
      if (src.kind == SV_LOGITS) {
        bad |= !(fabsf(v) <= 3.402823466e38f);
        a[i] = (double)v / src.T;
      } else {
        bad |= !(v >= 0.f && v <= 3.402823466e38f);
        a[i] = (double)v;
      }
      mx = fmax(mx, a[i]);
    }
  }
  double sum = 0.0;
  if (src.kind == SV_LOGITS) {
    mx = block_max_d(mx, sh);
#pragma unroll
    for (int i = 0; i < ACC_PER; ++i)
      if (x0 + threadIdx.x + 256 * i < V && !bad) sum += exp(a[i] - mx);
  } else {
    mx = 0.0;
#pragma unroll
    for (int i = 0; i < ACC_PER; ++i)
      if (x0 + threadIdx.x + 256 * i < V) sum += a[i];
  }
  sum = block_sum_d(sum, sh);
  bad = __any(bad) ? 1 : 0;
  if ((threadIdx.x & 63) == 0) shb[threadIdx.x >> 6] = bad;
  __syncthreads();
  if (threadIdx.x == 0) {
    const size_t o = (size_t)r * CH + c;
    ws.cmax[o] = mx;
    ws.csum[o] = sum;
    ws.cbad[o] = shb[0] | shb[1] | shb[2] | shb[3];
  }
}

// Distribution value of entry x of a row, given its recombined statistics.
__device__ inline double dist_val(const RowSrc& s, double m, double z, int x) {
  const float v = s.p[x];
  if (s.kind == SV_LOGITS) return exp((double)v / s.T - m) / z;
  return (double)v;
}

enum { MODE_RESID = 0, MODE_P = 1 };

__device__ inline double sample_weight(int mode, const RowSrc& P, double pm, double pz,
                                       const RowSrc& Q, double qm, double qz, int x) {
  const double p = dist_val(P, pm, pz, x);
  if (mode != MODE_RESID) return p;
  const double q = dist_val(Q, qm, qz, x);
  return fmax(p - q, 0.0);
}

// The row pair a sequence samples from, once n accepted drafts are known.
__device__ inline void sample_rows(int s, int n, int S, int K, int V, const float* target,
                                   int tkind, float Tp, const float* draft, int dkind, float Tq,
                                   RowSrc& P, RowSrc& Q) {
  P = row_src(s * (K + 1) + n, S, K, V, target, tkind, Tp, draft, dkind, Tq);
  Q = n < K ? row_src(S * (K + 1) + s * K + n, S, K, V, target, tkind, Tp, draft, dkind, Tq) : P;
}

__global__ __launch_bounds__(256) void k_acc_chunk(int S, int K, int V, const float* target,
                                                   int tkind, float Tp, const float* draft,
                                                   int dkind, float Tq, const int32_t* drafts,
                                                   const float* uni, AccWs ws) {
  __shared__ double rm[2 * SV_MAX_DRAFTS + 1], rz[2 * SV_MAX_DRAFTS + 1];
  __shared__ int rbad[2 * SV_MAX_DRAFTS + 1];
  __shared__ int s_nacc, s_invalid;
  __shared__ double sh[4];
  const int c = blockIdx.x, s = blockIdx.y, CH = gridDim.x;
  const int nrows = 2 * K + 1;
  const int tid = threadIdx.x;
  // 1. recombine the sequence's row statistics: wave w takes rows w, w+4, ...,
  //    lane l chunks l, l+64, ...; butterfly reductions, so the order (and
  //    the result) is the same in every block
  {
    const int lane = tid & 63, wv = tid >> 6;
    for (int i = wv; i < nrows; i += 4) {
      const int r = i <= K ? s * (K + 1) + i : S * (K + 1) + s * K + (i - K - 1);
      const bool logits = (i <= K ? tkind : dkind) == SV_LOGITS;
      double m = -INFINITY;
      int bad = 0;
      for (int cc = lane; cc < CH; cc += 64) {
        m = fmax(m, ws.cmax[(size_t)r * CH + cc]);
        bad |= ws.cbad[(size_t)r * CH + cc];
      }
      m = logits ? wave_max_d(m) : 0.0;
      bad = __any(bad) ? 1 : 0;
      double z = 0.0;
      for (int cc = lane; cc < CH; cc += 64) {
        const double cs = ws.csum[(size_t)r * CH + cc];
        z += logits ? cs * exp(ws.cmax[(size_t)r * CH + cc] - m) : cs;
      }
      z = wave_sum_d(z);
      if (lane == 0) {
        rm[i] = m;
        rz[i] = z;
        rbad[i] = bad | (logits ? 0 : !(z > 0.0));
      }
    }
  }
  __syncthreads();
  // 2. validity and 3. the accept chain: wave 0 tests every draft at once
  //    (lane i: draft i), the chain stops at the first rejection
  if (tid < 64) {
    int inv = 0;
    for (int i = tid; i < nrows; i += 64) inv |= rbad[i];
    for (int i = tid; i < K; i += 64) {
      const int d = drafts[s * K + i];
      inv |= !(d >= 0 && d < V);
    }
    for (int i = tid; i <= K; i += 64) {
      const float u = uni[s * (K + 1) + i];
      inv |= !(u >= 0.f && u < 1.f);
    }
    inv = __any(inv) ? 1 : 0;
    int rej = 0;   // this lane's draft is rejected (lanes past K: rejected)
    if (!inv) {
      rej = 1;
      if (tid < K) {
        const int d = drafts[s * K + tid];
        RowSrc P, Q;
        sample_rows(s, tid, S, K, V, target, tkind, Tp, draft, dkind, Tq, P, Q);
        const double p = dist_val(P, rm[tid], rz[tid], d);
        const double q = dist_val(Q, rm[K + 1 + tid], rz[K + 1 + tid], d);
        const double u = (double)uni[s * (K + 1) + tid];
        rej = !(fma(u, q, -p) < 0.0);   // reject: u*q >= p
      }
    }
    const unsigned long long rmask = __ballot(rej);
    const int n = inv ? 0 : (int)__builtin_ctzll(rmask);   // lanes >= K always reject (K <= 31)
    if (tid == 0) {
      s_nacc = n;
      s_invalid = inv;
      if (c == 0) {
        ws.sinfo[2 * s] = n;
        ws.sinfo[2 * s + 1] = inv;
        ws.sst[4 * s + 0] = rm[n];
        ws.sst[4 * s + 1] = rz[n];
        ws.sst[4 * s + 2] = n < K ? rm[K + 1 + n] : 0.0;
        ws.sst[4 * s + 3] = n < K ? rz[K + 1 + n] : 1.0;
      }
    }
  }
  __syncthreads();
  const int nacc = s_nacc;
  // 4. this chunk's total sampling weight (residual, or p_K for the bonus)
  RowSrc P, Q;
  sample_rows(s, nacc, S, K, V, target, tkind, Tp, draft, dkind, Tq, P, Q);
  const double pm = rm[nacc], pz = rz[nacc];
  const double qm = nacc < K ? rm[K + 1 + nacc] : 0.0, qz = nacc < K ? rz[K + 1 + nacc] : 1.0;
  const int mode = nacc < K ? MODE_RESID : MODE_P;
  double w = 0.0;
  if (!s_invalid) {
    const int x0 = c * ACC_CHUNK;
#pragma unroll
    for (int i = 0; i < ACC_PER; ++i) {
      const int x = x0 + tid * ACC_PER + i;
      if (x < V) w += sample_weight(mode, P, pm, pz, Q, qm, qz, x);
    }
  }
  w = block_sum_d(w, sh);
  if (tid == 0) ws.rsum[(size_t)s * CH + c] = w;
}

__global__ __launch_bounds__(256) void k_acc_pick(int S, int K, int V, int CH,
                                                  const float* target, int tkind, float Tp,
                                                  const float* draft, int dkind, float Tq,
                                                  const int32_t* drafts, const float* uni,
                                                  int32_t* out_tokens, int32_t* out_n, AccWs ws) {
  __shared__ double sh[4];
  __shared__ double s_base;
  __shared__ int s_hit, s_pick, s_last;
  const int s = blockIdx.x, tid = threadIdx.x;
  const int nacc = ws.sinfo[2 * s], invalid = ws.sinfo[2 * s + 1];
  int32_t* out = out_tokens + (size_t)s * (K + 1);
  if (invalid) {
    for (int i = tid; i <= K; i += 256) out[i] = -1;
    if (tid == 0) out_n[s] = -1;
    return;
  }
  RowSrc P, Q;
  sample_rows(s, nacc, S, K, V, target, tkind, Tp, draft, dkind, Tq, P, Q);
  const double pm = ws.sst[4 * s], pz = ws.sst[4 * s + 1], qm = ws.sst[4 * s + 2],
               qz = ws.sst[4 * s + 3];
  int mode = nacc < K ? MODE_RESID : MODE_P;
  double cw = tid < CH ? ws.rsum[(size_t)s * CH + tid] : 0.0;
  double Z;
  double pre = block_excl_scan_d(cw, sh, &Z);
  if (!(Z > 0.0)) {
    // the residual vanished (only through rounding): sample p_i itself
    mode = MODE_P;
    cw = 0.0;
    for (int cc = 0; cc < CH; ++cc) {
      double t = 0.0;
#pragma unroll
      for (int i = 0; i < ACC_PER; ++i) {
        const int x = cc * ACC_CHUNK + tid * ACC_PER + i;
        if (x < V) t += sample_weight(mode, P, pm, pz, Q, qm, qz, x);
      }
      t = block_sum_d(t, sh);
      if (tid == cc) cw = t;
    }
    pre = block_excl_scan_d(cw, sh, &Z);
  }
  const double target_t = (double)uni[s * (K + 1) + K] * Z;
  // chunk holding the target: the first whose running total exceeds it
  if (tid == 0) {
    s_hit = 0x7fffffff;
    s_last = -1;
    s_pick = 0x7fffffff;
  }
  __syncthreads();
  if (tid < CH && pre + cw > target_t) atomicMin(&s_hit, tid);
  if (tid < CH && cw > 0.0) atomicMax(&s_last, tid);
  __syncthreads();
  const bool found_chunk = s_hit != 0x7fffffff;
  // no chunk crossed (rounding): fall back to the last chunk with weight
  const int hit = found_chunk ? s_hit : (s_last >= 0 ? s_last : 0);
  if (tid == hit) s_base = pre;   // exclusive prefix of chunk `hit`
  __syncthreads();
  const double base = found_chunk ? s_base : 0.0;
  // in-chunk scan, 8 consecutive entries per thread
  double loc[ACC_PER];
  double tot = 0.0;
  int lastmine = -1;
#pragma unroll
  for (int i = 0; i < ACC_PER; ++i) {
    const int x = hit * ACC_CHUNK + tid * ACC_PER + i;
    loc[i] = x < V ? sample_weight(mode, P, pm, pz, Q, qm, qz, x) : 0.0;
    tot += loc[i];
    if (loc[i] > 0.0) lastmine = x;
  }
  double dummy;
  double run = base + block_excl_scan_d(tot, sh, &dummy);
  int mine = 0x7fffffff;
#pragma unroll
  for (int i = 0; i < ACC_PER; ++i) {
    run += loc[i];
    if (found_chunk && mine == 0x7fffffff && run > target_t) mine = hit * ACC_CHUNK + tid * ACC_PER + i;
  }
  __syncthreads();
  if (tid == 0) s_last = -1;
  __syncthreads();
  if (mine != 0x7fffffff) atomicMin(&s_pick, mine);
  if (lastmine >= 0) atomicMax(&s_last, lastmine);
  __syncthreads();
  if (tid == 0) {
    // none crossed (rounding): the last positive entry of the chunk
    const int tok = s_pick != 0x7fffffff ? s_pick : s_last;
    for (int i = 0; i < nacc; ++i) out[i] = drafts[s * K + i];
    out[nacc] = tok;
    for (int i = nacc + 1; i <= K; ++i) out[i] = -1;
    out_n[s] = nacc;
  }
}

hipError_t launch_accept(int S, int K, int V, const float* target, int tkind, float Tp,
                         const float* draft, int dkind, float Tq, const int32_t* drafts,
                         const float* u, int32_t* out_tokens, int32_t* out_n, void* wsp,
                         hipStream_t s) {
  const AccWs ws = acc_carve(wsp, S, K, V);
  const int CH = acc_chunks(V);
  hipLaunchKernelGGL(k_acc_stats, dim3(CH, S * (2 * K + 1)), dim3(256), 0, s, S, K, V, target,
                     tkind, Tp, draft, dkind, Tq, ws);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_acc_chunk, dim3(CH, S), dim3(256), 0, s, S, K, V, target, tkind, Tp, draft,
                     dkind, Tq, drafts, u, ws);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_acc_pick, dim3(S), dim3(256), 0, s, S, K, V, CH, target, tkind, Tp, draft,
                     dkind, Tq, drafts, u, out_tokens, out_n, ws);
  return hipGetLastError();
}

}  // namespace sv

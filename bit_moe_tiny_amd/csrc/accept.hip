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
// Target-sample matching (the second rule, "1x Spark tuned DSpark for
// DeepSeek-V4-Flash", the losslessness paragraph): every verify row's own
// inverse-CDF sample at its uniform; drafts stand while they equal these
// samples, the first that differs (or row K's) is emitted last.
//
// Three launches for the p/q rule, two for target-sample matching; no host
// sync, no block waiting on another:
//   k_acc_stats   grid (chunk, row): per 2048-entry chunk of every target and
//                 draft row, the chunk max of z/T and sum exp(z/T - max) in
//                 fp64 (or the plain sum for probability rows), plus a
//                 validity flag.  Spreads the vocabulary-wide reductions over
//                 many CUs.
//   k_acc_sample  grid (512-entry chunk, sequence): every block recombines
//                 its sequence's row statistics (same order in every block, so
//                 all agree bit for bit), replays the accept chain, and sums
//                 the sampling weights of its chunk (residual, or p_K for the
//                 bonus), per 2-entry thread segment and per chunk; block 0
//                 also stores the sequence's decision (accepted drafts, u_K,
//                 the sampled rows' statistics).
//   k_acc_pick    one block per sequence: from those sums (published by the
//                 kernel boundary, which costs less than a device-scope
//                 release and counter per block) it finds the chunk that
//                 holds u_K * Z, the segment inside it, and the token among
//                 that segment's entries, then writes the outputs.
//   k_tsm_pick    (target-sample matching) one block per target row: the
//                 row's masses per statistics chunk (its chunk sums rescaled
//                 to the row maximum) locate the chunk holding u Z, the block
//                 finds the token among that chunk's 2048 entries; the last
//                 row of a sequence to be sampled takes the prefix of
//                 matching drafts and writes the outputs.
#include "sv_internal.h"

namespace sv {

constexpr int ACC_T = 256;                    // threads per block
constexpr int ACC_CHUNK = 2048;               // statistics chunk
// threads per statistics block: 1024 for grids of fewer than STATS_WIDE
// blocks (short per-thread chains), 256 beyond (more blocks per CU)
constexpr int STATS_WIDE = 512;
constexpr int ACC_MAX_CH = 256;               // V <= 524288
constexpr int SMP_PER = 2;                    // sampling entries per thread
constexpr int SMP_CHUNK = ACC_T * SMP_PER;    // sampling chunk
constexpr int SMP_MAX_CH = ACC_MAX_CH * ACC_CHUNK / SMP_CHUNK;

// A logits row at temperature 0 (greedy decoding): the one-hot distribution at
// the row's first largest value.  Its statistics are the maximum and, in place
// of the softmax denominator, that value's index.
constexpr int ACC_ARGMAX = 2;

struct AccWs {
  double* cmax;     // [rows, CH]
  double* csum;     // [rows, CH]
  int* cbad;        // [rows, CH]
  double* rsum;     // [S, CHs]        sampling weight per sampling chunk
  double* tsum;     // [S, CHs, ACC_T] sampling weight per thread segment
  unsigned* done;   // [S]            (target-sample matching only) rows sampled
  int* sdec;        // [S, 2]         accepted drafts, invalid flag
  double* sst;      // [S, 5]         u_K and the sampled rows' statistics pm, pz, qm, qz
};

static inline int acc_chunks(int V) { return (V + ACC_CHUNK - 1) / ACC_CHUNK; }
static inline int smp_chunks(int V) { return (V + SMP_CHUNK - 1) / SMP_CHUNK; }

static AccWs acc_carve(void* base, int S, int K, int V) {
  const size_t rows = (size_t)S * (2 * K + 1), CH = acc_chunks(V), CHs = smp_chunks(V);
  uint8_t* p = (uint8_t*)base;
  AccWs w;
  w.cmax = (double*)p;
  p += up256(rows * CH * 8);
  w.csum = (double*)p;
  p += up256(rows * CH * 8);
  w.cbad = (int*)p;
  p += up256(rows * CH * 4);
  w.rsum = (double*)p;
  p += up256((size_t)S * CHs * 8);
  w.tsum = (double*)p;
  p += up256((size_t)S * CHs * ACC_T * 8);
  w.done = nullptr;
  w.sdec = (int*)p;
  p += up256((size_t)S * 8);
  w.sst = (double*)p;
  return w;
}

size_t accept_ws_bytes(int S, int K, int V) {
  const size_t rows = (size_t)S * (2 * K + 1), CH = acc_chunks(V), CHs = smp_chunks(V);
  return 2 * up256(rows * CH * 8) + up256(rows * CH * 4) + up256((size_t)S * CHs * 8) +
         up256((size_t)S * CHs * ACC_T * 8) + up256((size_t)S * 8) + up256((size_t)S * 40);
}

__device__ inline double wave_sum_d(double v) {
  return wave_allreduce(v, [](double a, double b) { return a + b; });
}
__device__ inline double wave_max_d(double v) {
  return wave_allreduce(v, [](double a, double b) { return fmax(a, b); });
}

// x from the lane CTRL names (DPP), 0 where the row/bank masks or the row
// edge leave no source: 0x111/0x112/0x114/0x118 row_shr 1/2/4/8, 0x142
// row_bcast 15, 0x143 row_bcast 31.
template <int CTRL, int ROWS, int BANKS>
__device__ __forceinline__ double xlane_z(double x) {
  const uint64_t b = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, ROWS, BANKS, true);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, ROWS, BANKS, true);
  return __builtin_bit_cast(double, (uint64_t)lo | ((uint64_t)hi << 32));
}

// Wave-wide exclusive prefix sum in a fixed order (inclusive scan in 16-lane
// rows by row shifts, then the row totals broadcast across rows);
// *total = the wave's sum.
__device__ inline double wave_excl_scan_d(double v, double* total) {
  double x = v;
  x += xlane_z<0x111, 0xF, 0xF>(x);
  x += xlane_z<0x112, 0xF, 0xF>(x);
  x += xlane_z<0x114, 0xF, 0xE>(x);
  x += xlane_z<0x118, 0xF, 0xC>(x);
  x += xlane_z<0x142, 0xA, 0xF>(x);
  x += xlane_z<0x143, 0xC, 0xF>(x);
  const uint64_t b = __builtin_bit_cast(uint64_t, x);
  *total = __builtin_bit_cast(double, (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, 63) |
                                          ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), 63) << 32));
  const double ex = __shfl_up(x, 1, 64);
  return (threadIdx.x & 63) == 0 ? 0.0 : ex;
}

// Block-wide fixed-order reductions over NW waves (the per-wave results
// folded left in wave order); `sh` holds NW doubles.
template <int NW = ACC_T / 64>
__device__ inline double block_sum_d(double v, double* sh) {
  v = wave_sum_d(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  double t = sh[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) t += sh[w];
  return t;
}
template <int NW = ACC_T / 64>
__device__ inline double block_max_d(double v, double* sh) {
  v = wave_max_d(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  double t = sh[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) t = fmax(t, sh[w]);
  return t;
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
  double rT;        // 1 / T: z / T is taken as z * rT everywhere
};

__device__ inline RowSrc row_src(int r, int S, int K, int V, const float* target, int tkind,
                                 float Tp, const float* draft, int dkind, float Tq) {
  RowSrc s;
  const int nt = S * (K + 1);
  if (r < nt) {
    s.p = target + (size_t)r * V;
    s.kind = tkind;
    s.rT = 1.0 / (double)Tp;
  } else {
    s.p = draft + (size_t)(r - nt) * V;
    s.kind = dkind;
    s.rT = 1.0 / (double)Tq;
  }
  return s;
}

template <int STATS_T>
__global__ __launch_bounds__(STATS_T) void k_acc_stats(int S, int K, int V, const float* target,
                                                   int tkind, float Tp, const float* draft,
                                                   int dkind, float Tq, AccWs ws, int n_clear) {
  constexpr int NW = STATS_T / 64, STATS_PER = ACC_CHUNK / STATS_T;
  __shared__ double sh[NW];
  __shared__ int shb[NW];
  const int c = blockIdx.x, r = blockIdx.y, CH = gridDim.x;
  if (c == 0 && r == 0)   // target-sample matching: its per-sequence counters
    for (int i = threadIdx.x; i < n_clear; i += blockDim.x) ws.done[i] = 0u;
  const RowSrc src = row_src(r, S, K, V, target, tkind, Tp, draft, dkind, Tq);
  const int x0 = c * ACC_CHUNK;
  double a[STATS_PER];
  int bad = 0;
  double mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < STATS_PER; ++i) {
    const int x = x0 + threadIdx.x + STATS_T * i;
    a[i] = -INFINITY;
    if (x < V) {
      const float v = src.p[x];
      if (src.kind != SV_PROBS) {
        bad |= !(fabsf(v) <= 3.402823466e38f);
        a[i] = src.kind == SV_LOGITS ? (double)v * src.rT : (double)v;
      } else {
        bad |= !(v >= 0.f && v <= 3.402823466e38f);
        a[i] = (double)v;
      }
      mx = fmax(mx, a[i]);
    }
  }
  double sum = 0.0;
  if (src.kind == SV_LOGITS) {
    mx = block_max_d<NW>(mx, sh);
#pragma unroll
    for (int i = 0; i < STATS_PER; ++i)
      if (x0 + threadIdx.x + STATS_T * i < V && !bad) sum += exp(a[i] - mx);
    sum = block_sum_d<NW>(sum, sh);
  } else if (src.kind == ACC_ARGMAX) {
    // the chunk's first index holding its maximum (a maximum of -index)
    mx = block_max_d<NW>(mx, sh);
    double fi = -INFINITY;
#pragma unroll
    for (int i = STATS_PER - 1; i >= 0; --i)
      if (x0 + threadIdx.x + STATS_T * i < V && a[i] == mx) fi = -(double)(x0 + threadIdx.x + STATS_T * i);
    sum = -block_max_d<NW>(fi, sh);
  } else {
    mx = 0.0;
#pragma unroll
    for (int i = 0; i < STATS_PER; ++i)
      if (x0 + threadIdx.x + STATS_T * i < V) sum += a[i];
    sum = block_sum_d<NW>(sum, sh);
  }
  bad = __any(bad) ? 1 : 0;
  if ((threadIdx.x & 63) == 0) shb[threadIdx.x >> 6] = bad;
  __syncthreads();
  if (threadIdx.x == 0) {
    const size_t o = (size_t)r * CH + c;
    ws.cmax[o] = mx;
    ws.csum[o] = sum;
    int cb = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) cb |= shb[w];
    ws.cbad[o] = cb;
  }
}

static void launch_acc_stats(dim3 grid, hipStream_t s, int S, int K, int V, const float* target, int tkind,
                             float Tp, const float* draft, int dkind, float Tq, AccWs ws, int n_clear) {
  if (grid.x * grid.y < (unsigned)STATS_WIDE)
    hipLaunchKernelGGL(k_acc_stats<1024>, grid, dim3(1024), 0, s, S, K, V, target, tkind, Tp, draft, dkind, Tq,
                       ws, n_clear);
  else
    hipLaunchKernelGGL(k_acc_stats<256>, grid, dim3(256), 0, s, S, K, V, target, tkind, Tp, draft, dkind, Tq, ws,
                       n_clear);
}

// Distribution value of entry x of a row, given its recombined statistics.
__device__ inline double dist_val(const RowSrc& s, double m, double z, int x) {
  if (s.kind == ACC_ARGMAX) return x == (int)z ? 1.0 : 0.0;
  const float v = s.p[x];
  if (s.kind == SV_LOGITS) return exp((double)v * s.rT - m) / z;
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

// One row's statistics from lane-held chunk statistics (lane l: chunks l,
// l + 64, ...): the maximum and the softmax denominator rescaled to it (the
// plain sum for probability rows; for a greedy row the first index holding
// the maximum), fixed-order butterfly reductions.
template <int CPL>
__device__ inline void row_reduce(const double (&cm)[CPL], const double (&cs)[CPL], int CH, int kind,
                                  double* m_out, double* z_out) {
  const int lane = threadIdx.x & 63;
  double m = -INFINITY;
#pragma unroll
  for (int k = 0; k < CPL; ++k) m = fmax(m, cm[k]);
  m = kind != SV_PROBS ? wave_max_d(m) : 0.0;
  double z = 0.0;
  if (kind == ACC_ARGMAX) {
    // the first chunk holding the row's maximum gives the index
    double f = -INFINITY;
#pragma unroll
    for (int k = 0; k < CPL; ++k)
      if (lane + 64 * k < CH && cm[k] == m) f = fmax(f, -cs[k]);
    z = -wave_max_d(f);
  } else {
#pragma unroll
    for (int k = 0; k < CPL; ++k)
      if (lane + 64 * k < CH) z += kind == SV_LOGITS ? cs[k] * exp(cm[k] - m) : cs[k];
    z = wave_sum_d(z);
  }
  *m_out = m;
  *z_out = z;
}

// Row statistics of sequence s recombined from the chunk statistics: wave w
// takes rows w, w+4, ... three at a time (their loads issued together), lane
// l chunks l, l+64, ...; butterfly reductions, so every block gets the same
// bits.
__device__ inline void acc_rows(int s, int S, int K, int CH, int tkind, int dkind, const AccWs& ws,
                                double* rm, double* rz, int* rbad) {
  constexpr int RB = 3, CPL = ACC_MAX_CH / 64;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int nrows = 2 * K + 1;
  for (int i0 = wv; i0 < nrows; i0 += 4 * RB) {
    double cm[RB][CPL], cs[RB][CPL];
    int cb[RB];
#pragma unroll
    for (int j = 0; j < RB; ++j) {
      const int i = i0 + 4 * j;
      const int r = i <= K ? s * (K + 1) + i : S * (K + 1) + s * K + (i - K - 1);
      cb[j] = 0;
#pragma unroll
      for (int k = 0; k < CPL; ++k) {
        const int cc = lane + 64 * k;
        cm[j][k] = -INFINITY;
        cs[j][k] = 0.0;
        if (i < nrows && cc < CH) {
          const size_t o = (size_t)r * CH + cc;
          cm[j][k] = ws.cmax[o];
          cs[j][k] = ws.csum[o];
          cb[j] |= ws.cbad[o];
        }
      }
    }
#pragma unroll
    for (int j = 0; j < RB; ++j) {
      const int i = i0 + 4 * j;
      if (i >= nrows) break;   // uniform in the wave
      const int kind = i <= K ? tkind : dkind;
      double m, z;
      row_reduce<CPL>(cm[j], cs[j], CH, kind, &m, &z);
      const int bad = __any(cb[j]) ? 1 : 0;
      if (lane == 0) {
        rm[i] = m;
        rz[i] = z;
        rbad[i] = bad | (kind == SV_PROBS ? !(z > 0.0) : 0);
      }
    }
  }
}

// Sampling weight of this thread's segment of sampling chunk c: entries
// c*SMP_CHUNK + tid*SMP_PER + 0..SMP_PER-1, summed in order.
__device__ inline double seg_weight(int mode, const RowSrc& P, double pm, double pz,
                                    const RowSrc& Q, double qm, double qz, int c, int V) {
  double w = 0.0;
#pragma unroll
  for (int i = 0; i < SMP_PER; ++i) {
    const int x = c * SMP_CHUNK + threadIdx.x * SMP_PER + i;
    if (x < V) w += sample_weight(mode, P, pm, pz, Q, qm, qz, x);
  }
  return w;
}

// Running sums over n values v[0..n) in LDS, in order (lane l holds
// v[l*per .. l*per+per-1]).  wave_prefix: the lane's exclusive prefix and
// the total.  wave_cross: the first index at which the running sum from
// `run` (the lane's starting sum) exceeds tt, and the running sum before it
// (-1 if none); *lastpos = the last index with a positive value (-1 if none).
// Wave-uniform results.
__device__ inline double wave_prefix(const double* v, int n, int per, double* total) {
  const int lane = threadIdx.x & 63;
  double lt = 0.0;
  for (int j = 0; j < per; ++j) {
    const int k = lane * per + j;
    if (k < n) lt += v[k];
  }
  return wave_excl_scan_d(lt, total);
}

__device__ inline int wave_cross(const double* v, int n, int per, double run, double tt, double* pre,
                                 int* lastpos) {
  const int lane = threadIdx.x & 63;
  int cand = -1, lp = -1;
  double cpre = 0.0;
  for (int j = 0; j < per; ++j) {
    const int k = lane * per + j;
    if (k < n) {
      const double x = v[k];
      if (cand < 0 && run + x > tt) {
        cand = k;
        cpre = run;
      }
      if (x > 0.0) lp = k;
      run += x;
    }
  }
  const unsigned long long cm = __ballot(cand >= 0), pmask = __ballot(lp >= 0);
  *lastpos = pmask ? __shfl(lp, 63 - __builtin_clzll(pmask), 64) : -1;
  if (!cm) return -1;
  const int fl = __builtin_ctzll(cm);
  *pre = __shfl(cpre, fl, 64);
  return __shfl(cand, fl, 64);
}

// The sampled chunk, run by the block whose LDS holds the chunk totals
// cws[0..CHs): wave 0 finds the first chunk whose running total exceeds
// tt = u Z, failing that (rounding) the last chunk with weight.  Sets *z
// (the total Z), *found, *hit and *base (the running total before the hit
// chunk); ends with a block barrier.
__device__ inline void find_chunk(const double* cws, int CHs, double u, double* z, int* found, int* hit,
                                  double* base) {
  if (threadIdx.x < 64) {
    const int per = (CHs + 63) / 64;
    double Z;
    const double run = wave_prefix(cws, CHs, per, &Z);
    double pre = 0.0;
    int lastpos = -1;
    const int h = Z > 0.0 ? wave_cross(cws, CHs, per, run, u * Z, &pre, &lastpos) : -1;
    if ((threadIdx.x & 63) == 0) {
      *z = Z;
      *found = h >= 0;
      *hit = h >= 0 ? h : max(lastpos, 0);
      *base = h >= 0 ? pre : 0.0;
    }
  }
  __syncthreads();
}

// The sampled entry of chunk `hit`, by wave 0, given the per-thread segment
// weights parts[0..ACC_T) of that chunk in LDS: the thread segment whose
// running sum (from base) first exceeds tt, then the entry inside it, failing
// that (rounding) the last entry with weight of the segment, of the chunk.
template <int PER = SMP_PER>
__device__ inline int seg_token(const double* parts, double base, bool found_chunk, double tt, int hit,
                                int mode, const RowSrc& P, double pm, double pz, const RowSrc& Q, double qm,
                                double qz, int V) {
  const int lane = threadIdx.x & 63;
  constexpr int TPL = ACC_T / 64, CHUNK = ACC_T * PER;
  double ptot;
  const double prun = base + wave_prefix(parts, ACC_T, TPL, &ptot);
  double tpre = 0.0;
  int lastseg;
  const int seg = wave_cross(parts, ACC_T, TPL, prun, tt, &tpre, &lastseg);
  const bool found = found_chunk && seg >= 0;
  const int thr = found ? seg : max(lastseg, 0);
  int tok = -1;
  {
    double run = tpre;
    int lp = -1;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int x = hit * CHUNK + thr * PER + i;
      if (x < V) {
        const double wi = sample_weight(mode, P, pm, pz, Q, qm, qz, x);
        run += wi;
        if (wi > 0.0) lp = x;
        if (found && tok < 0 && run > tt) tok = x;
      }
    }
    if (tok < 0) tok = lp;
  }
  if (tok < 0) {
    // (rounding put the crossing in a segment without weight) the chunk's
    // last entry with weight
    int lp = -1;
    for (int i = lane; i < CHUNK; i += 64) {
      const int x = hit * CHUNK + i;
      if (x < V && sample_weight(mode, P, pm, pz, Q, qm, qz, x) > 0.0) lp = x;
    }
    for (int o = 32; o >= 1; o >>= 1) lp = max(lp, __shfl_xor(lp, o, 64));
    tok = lp;
  }
  return tok;
}

__global__ __launch_bounds__(ACC_T) void k_acc_sample(int S, int K, int V, int CH,
                                                      const float* target, int tkind, float Tp,
                                                      const float* draft, int dkind, float Tq,
                                                      const int32_t* drafts, const float* uni, AccWs ws) {
  __shared__ double rm[2 * SV_MAX_DRAFTS + 1], rz[2 * SV_MAX_DRAFTS + 1];
  __shared__ int rbad[2 * SV_MAX_DRAFTS + 1];
  __shared__ double sh[4];
  __shared__ double s_uk;
  __shared__ int s_nacc, s_invalid;
  const int c = blockIdx.x, s = blockIdx.y, CHs = gridDim.x;
  const int tid = threadIdx.x, lane = tid & 63;
  // 0. wave 0, lane i: draft i's token and uniform and both rows' values at
  //    the token, loaded before the statistics are read
  int dk = -1, pre_bad = 0;
  float uk = 0.f, vp = 0.f, vq = 0.f;
  if (tid < 64) {
    if (lane <= K) {
      uk = uni[s * (K + 1) + lane];
      pre_bad |= !(uk >= 0.f && uk < 1.f);
    }
    if (lane < K) {
      dk = drafts[s * K + lane];
      if (dk >= 0 && dk < V) {
        vp = target[(size_t)(s * (K + 1) + lane) * V + dk];
        vq = draft[(size_t)(s * K + lane) * V + dk];
      } else {
        pre_bad = 1;
      }
    }
  }
  // 1. the sequence's row statistics
  acc_rows(s, S, K, CH, tkind, dkind, ws, rm, rz, rbad);
  __syncthreads();
  // 2. validity and the accept chain: wave 0 tests every draft at once
  //    (lane i: draft i), the chain stops at the first rejection
  if (tid < 64) {
    int inv = pre_bad;
    for (int i = lane; i < 2 * K + 1; i += 64) inv |= rbad[i];
    inv = __any(inv) ? 1 : 0;
    int rej = 1;   // lanes past K: rejected (K <= 31)
    if (!inv && lane < K) {
      const double p = tkind == SV_LOGITS    ? exp((double)vp * (1.0 / (double)Tp) - rm[lane]) / rz[lane]
                       : tkind == ACC_ARGMAX ? (dk == (int)rz[lane] ? 1.0 : 0.0)
                                             : (double)vp;
      const double q = dkind == SV_LOGITS ? exp((double)vq * (1.0 / (double)Tq) - rm[K + 1 + lane]) / rz[K + 1 + lane]
                       : dkind == ACC_ARGMAX ? (dk == (int)rz[K + 1 + lane] ? 1.0 : 0.0)
                                             : (double)vq;
      rej = !(fma((double)uk, q, -p) < 0.0);   // reject: u*q >= p
    }
    const unsigned long long rmask = __ballot(rej);
    if (lane == 0) {
      s_nacc = inv ? 0 : (int)__builtin_ctzll(rmask);
      s_invalid = inv;
    }
    if (lane == K) s_uk = (double)uk;
  }
  __syncthreads();
  const int nacc = s_nacc, inv = s_invalid;
  // 3. this chunk's sampling weights (residual, or p_K for the bonus), per
  //    thread segment and per chunk
  RowSrc P, Q;
  sample_rows(s, nacc, S, K, V, target, tkind, Tp, draft, dkind, Tq, P, Q);
  const double pm = rm[nacc], pz = rz[nacc];
  const double qm = nacc < K ? rm[K + 1 + nacc] : 0.0, qz = nacc < K ? rz[K + 1 + nacc] : 1.0;
  const int mode = nacc < K ? MODE_RESID : MODE_P;
  double w = inv ? 0.0 : seg_weight(mode, P, pm, pz, Q, qm, qz, c, V);
  // 4. the chunk's sums for k_acc_pick (the kernel boundary publishes them),
  //    and, from block 0, the sequence's decision
  ws.tsum[((size_t)s * CHs + c) * ACC_T + tid] = w;
  w = block_sum_d(w, sh);
  if (tid == 0) ws.rsum[(size_t)s * CHs + c] = w;
  if (c == 0 && tid == 0) {
    ws.sdec[2 * s] = nacc;
    ws.sdec[2 * s + 1] = inv;
    double* st = ws.sst + 5 * (size_t)s;
    st[0] = s_uk;
    st[1] = pm;
    st[2] = pz;
    st[3] = qm;
    st[4] = qz;
  }
}

// One block per sequence: from the chunk totals, the chunk that holds
// u_K * Z, then the thread segment and the entry inside it (from the
// segment sums), and the sequence's outputs.
__global__ __launch_bounds__(ACC_T) void k_acc_pick(int S, int K, int V, const float* target, int tkind, float Tp,
                                                    const float* draft, int dkind, float Tq, const int32_t* drafts,
                                                    int CHs, int32_t* out_tokens, int32_t* out_n, AccWs ws) {
  __shared__ double sh[4];
  __shared__ double cws[SMP_MAX_CH];   // chunk totals
  __shared__ double parts[ACC_T];      // the hit chunk's segment totals
  __shared__ double s_z, s_base;
  __shared__ int s_hit, s_found;
  const int s = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const int nacc = ws.sdec[2 * s], inv = ws.sdec[2 * s + 1];
  const double* st = ws.sst + 5 * (size_t)s;
  const double uk = st[0], pm = st[1], pz = st[2], qm = st[3], qz = st[4];
  for (int cc = tid; cc < CHs; cc += ACC_T) cws[cc] = ws.rsum[(size_t)s * CHs + cc];
  const int dk = lane < K && lane < nacc ? drafts[s * K + lane] : -1;
  __syncthreads();
  int32_t* out = out_tokens + (size_t)s * (K + 1);
  if (inv) {
    if (tid <= K) out[tid] = -1;
    if (tid == 0) out_n[s] = -1;
    return;
  }
  RowSrc P, Q;
  sample_rows(s, nacc, S, K, V, target, tkind, Tp, draft, dkind, Tq, P, Q);
  const int mode = nacc < K ? MODE_RESID : MODE_P;
  // the chunk holding tt = u_K * Z
  find_chunk(cws, CHs, uk, &s_z, &s_found, &s_hit, &s_base);
  const bool redo = !(s_z > 0.0);
  if (redo) {
    // the residual vanished (only through rounding): sample p itself
    for (int cc = 0; cc < CHs; ++cc) {
      const double t = block_sum_d(seg_weight(MODE_P, P, pm, pz, Q, qm, qz, cc, V), sh);
      if (tid == 0) cws[cc] = t;
    }
    __syncthreads();
    find_chunk(cws, CHs, uk, &s_z, &s_found, &s_hit, &s_base);
  }
  const int smode = redo ? MODE_P : mode;
  const double tt = uk * s_z;
  const int hit = s_hit;
  parts[tid] = redo ? seg_weight(MODE_P, P, pm, pz, Q, qm, qz, hit, V)
                    : ws.tsum[((size_t)s * CHs + hit) * ACC_T + tid];
  __syncthreads();
  if (tid >= 64) return;
  // the thread segment inside it, then the entry
  const int tok = seg_token(parts, s_base, s_found, tt, hit, smode, P, pm, pz, Q, qm, qz, V);
  if (lane <= K) out[lane] = lane < nacc ? dk : (lane == nacc ? tok : -1);
  if (lane == 0) out_n[s] = nacc;
}

hipError_t launch_accept(int S, int K, int V, const float* target, int tkind, float Tp,
                         const float* draft, int dkind, float Tq, const int32_t* drafts,
                         const float* u, int32_t* out_tokens, int32_t* out_n, void* wsp,
                         hipStream_t s) {
  const AccWs ws = acc_carve(wsp, S, K, V);
  const int CH = acc_chunks(V), CHs = smp_chunks(V);
  if (tkind == SV_LOGITS && Tp == 0.f) tkind = ACC_ARGMAX;   // greedy rows
  if (dkind == SV_LOGITS && Tq == 0.f) dkind = ACC_ARGMAX;
  launch_acc_stats(dim3(CH, S * (2 * K + 1)), s, S, K, V, target, tkind, Tp, draft, dkind, Tq, ws, 0);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_acc_sample, dim3(CHs, S), dim3(ACC_T), 0, s, S, K, V, CH, target, tkind,
                     Tp, draft, dkind, Tq, drafts, u, ws);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_acc_pick, dim3(S), dim3(ACC_T), 0, s, S, K, V, target, tkind, Tp, draft, dkind, Tq, drafts,
                     CHs, out_tokens, out_n, ws);
  return hipGetLastError();
}

// ------------------------------------------------- target-sample matching
struct TsmWs {
  double* cmax;     // [rows, CH]
  double* csum;     // [rows, CH]
  int* cbad;        // [rows, CH]
  int* tok;         // [rows]  each row's sample (-1: invalid row or uniform)
  unsigned* done;   // [S]     rows of each sequence sampled
};

static TsmWs tsm_carve(void* base, int S, int K, int V) {
  const size_t rows = (size_t)S * (K + 1), CH = acc_chunks(V);
  uint8_t* p = (uint8_t*)base;
  TsmWs w;
  w.cmax = (double*)p;
  p += up256(rows * CH * 8);
  w.csum = (double*)p;
  p += up256(rows * CH * 8);
  w.cbad = (int*)p;
  p += up256(rows * CH * 4);
  w.tok = (int*)p;
  p += up256(rows * 4);
  w.done = (unsigned*)p;
  return w;
}

size_t accept_tsm_ws_bytes(int S, int K, int V) {
  const size_t rows = (size_t)S * (K + 1), CH = acc_chunks(V);
  return 2 * up256(rows * CH * 8) + up256(rows * CH * 4) + up256(rows * 4) + up256((size_t)S * 4);
}

// Row r's statistics from its chunk statistics, by wave 0 (the same
// reduction as the p/q rule's rows).
__device__ inline void tsm_row_stats(int r, int CH, int kind, const TsmWs& ws, double* m, double* z, int* bad) {
  constexpr int CPL = ACC_MAX_CH / 64;
  const int lane = threadIdx.x & 63;
  double cm[CPL], cs[CPL];
  int cb = 0;
#pragma unroll
  for (int k = 0; k < CPL; ++k) {
    const int cc = lane + 64 * k;
    cm[k] = -INFINITY;
    cs[k] = 0.0;
    if (cc < CH) {
      const size_t o = (size_t)r * CH + cc;
      cm[k] = ws.cmax[o];
      cs[k] = ws.csum[o];
      cb |= ws.cbad[o];
    }
  }
  row_reduce<CPL>(cm, cs, CH, kind, m, z);
  *bad = (__any(cb) ? 1 : 0) | (kind == SV_PROBS ? !(*z > 0.0) : 0);
}

__global__ __launch_bounds__(ACC_T) void k_tsm_pick(int S, int K, int V, int CH, const float* target,
                                                    int tkind, float Tp, const int32_t* drafts, const float* uni,
                                                    int32_t* out_tokens, int32_t* out_n, TsmWs ws) {
  __shared__ double cws[ACC_MAX_CH];   // the row's mass per statistics chunk
  __shared__ double parts[ACC_T];      // the hit chunk's mass per 8-entry thread segment
  __shared__ double s_m, s_zr, s_z, s_base;
  __shared__ int s_bad, s_hit, s_found;
  const int r = blockIdx.x, s = r / (K + 1), i = r - s * (K + 1);
  const int tid = threadIdx.x, lane = tid & 63;
  constexpr int PER = ACC_CHUNK / ACC_T;
  // 1. the row's statistics and its mass per chunk: the chunk sums rescaled
  //    to the row's maximum (unnormalised, like the entry weights below)
  if (tid < 64) {
    double m, z;
    int bad;
    tsm_row_stats(r, CH, tkind, ws, &m, &z, &bad);
    for (int c = lane; c < CH; c += 64) {
      const size_t o = (size_t)r * CH + c;
      cws[c] = tkind == SV_LOGITS ? ws.csum[o] * exp(ws.cmax[o] - m) : ws.csum[o];
    }
    if (lane == 0) {
      s_m = m;
      s_zr = z;
      s_bad = bad;
    }
  }
  __syncthreads();
  RowSrc P;
  P.p = target + (size_t)r * V;
  P.kind = tkind;
  P.rT = 1.0 / (double)Tp;
  // 2. row r's sample at u_i (block-uniform branches): a greedy row's token is
  //    its first maximum; otherwise the chunk holding u Z, then the entry
  const float uf = uni[(size_t)s * (K + 1) + i];
  const bool ok = !s_bad && uf >= 0.f && uf < 1.f;
  int tok = -1;
  if (ok && tkind == ACC_ARGMAX) {
    tok = (int)s_zr;
  } else if (ok) {
    find_chunk(cws, CH, (double)uf, &s_z, &s_found, &s_hit, &s_base);
    double w = 0.0;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int x = s_hit * ACC_CHUNK + tid * PER + e;
      if (x < V) w += sample_weight(MODE_P, P, s_m, 1.0, P, 0.0, 1.0, x);
    }
    parts[tid] = w;
    __syncthreads();
    if (tid < 64)
      tok = seg_token<PER>(parts, s_base, s_found, (double)uf * s_z, s_hit, MODE_P, P, s_m, 1.0, P, 0.0, 1.0, V);
  }
  if (tid >= 64) return;
  // 3. publish it (the same lane stores it and counts the row done with an
  //    acquire-release increment); the last row of the sequence to be
  //    sampled decides, after an acquire of its own wave
  unsigned prev = 0;
  if (lane == 0) {
    __hip_atomic_store(&ws.tok[r], tok, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    prev = __hip_atomic_fetch_add(&ws.done[s], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
  }
  prev = __builtin_amdgcn_readfirstlane(prev);
  if (prev != (unsigned)K) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  int ti = -1, di = -1, inv = 0;
  if (lane <= K) {
    ti = __hip_atomic_load(&ws.tok[s * (K + 1) + lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    inv |= ti < 0;
  }
  if (lane < K) {
    di = drafts[s * K + lane];
    inv |= !(di >= 0 && di < V);
  }
  inv = __any(inv) ? 1 : 0;
  // the first row whose sample differs from its draft (row K always "differs")
  const unsigned long long mism = __ballot(lane < K ? ti != di : 1);
  const int n = (int)__builtin_ctzll(mism);
  int32_t* out = out_tokens + (size_t)s * (K + 1);
  if (lane <= K) out[lane] = inv ? -1 : lane < n ? di : (lane == n ? ti : -1);
  if (lane == 0) out_n[s] = inv ? -1 : n;
}

hipError_t launch_accept_tsm(int S, int K, int V, const float* target, int tkind, float Tp,
                             const int32_t* drafts, const float* u, int32_t* out_tokens, int32_t* out_n,
                             void* wsp, hipStream_t s) {
  const TsmWs tw = tsm_carve(wsp, S, K, V);
  AccWs aw{};
  aw.cmax = tw.cmax;
  aw.csum = tw.csum;
  aw.cbad = tw.cbad;
  aw.done = tw.done;
  const int CH = acc_chunks(V), rows = S * (K + 1);
  if (tkind == SV_LOGITS && Tp == 0.f) tkind = ACC_ARGMAX;   // greedy rows
  // target rows only (row index < S (K+1)); no draft rows are read
  launch_acc_stats(dim3(CH, rows), s, S, K, V, target, tkind, Tp, (const float*)nullptr, tkind, Tp, aw, S);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_tsm_pick, dim3(rows), dim3(ACC_T), 0, s, S, K, V, CH, target, tkind, Tp, drafts, u,
                     out_tokens, out_n, tw);
  return hipGetLastError();
}

}  // namespace sv

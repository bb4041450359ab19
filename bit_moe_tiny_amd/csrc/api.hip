// C ABI of libspecverify: host-side validation, workspace carving and launch
// sequencing.  Nothing is enqueued unless every argument checks out.
#include <math.h>

#include <atomic>

#include "sv_internal.h"

using namespace sv;

namespace sv {

int cu_count() {
  constexpr int MAX_DEV = 64;
  static std::atomic<int> cache[MAX_DEV];   // 0 = not queried yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::atomic<int>* slot = dev >= 0 && dev < MAX_DEV ? &cache[dev] : nullptr;
  int n = slot ? slot->load(std::memory_order_relaxed) : 0;
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  if (slot) slot->store(n, std::memory_order_relaxed);
  return n;
}

}  // namespace sv

namespace {

constexpr int MAX_K_STAGE = 16384;   // activation staging keeps one row in LDS

bool dtype_ok(int t) { return t == SV_F32 || t == SV_BF16; }
bool kind_ok(int t) { return t == SV_LOGITS || t == SV_PROBS; }

int moe_check(const sv_moe_desc* d, int R) {
  if (!d || R < 1 || R > SV_MAX_ROWS) return SV_EINVAL;
  if (d->hidden < 256 || d->hidden % 256 || d->hidden > MAX_K_STAGE) return SV_EINVAL;
  if (d->ffn == SV_FFN_PLAIN) {
    if (d->inter < 1 || d->n_experts != 1 || d->top_k != 1 || !d->w_gate) return SV_EINVAL;
    if (d->w_up || d->w_down || d->s_gate || d->s_up || d->s_down) return SV_EINVAL;
    return SV_OK;
  }
  if (d->ffn != SV_FFN_SWIGLU) return SV_EINVAL;
  if (d->inter < 256 || d->inter % 256 || d->inter > MAX_K_STAGE) return SV_EINVAL;
  if (d->n_experts < 1 || d->n_experts > SV_MAX_EXPERTS) return SV_EINVAL;
  if (d->top_k < 1 || d->top_k > SV_MAX_TOPK || d->top_k > d->n_experts) return SV_EINVAL;
  if (!d->w_gate || !d->w_up || !d->w_down) return SV_EINVAL;
  const int ns = (d->s_gate != nullptr) + (d->s_up != nullptr) + (d->s_down != nullptr);
  if (ns != 0 && ns != 3) return SV_EINVAL;
  if (ns == 3 && d->s_format != SV_Q2 && d->s_format != SV_Q8) return SV_EINVAL;
  return SV_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? SV_OK : SV_EHIP; }

}  // namespace

extern "C" {

int sv_api_version(void) { return SV_API_VERSION; }

const char* sv_status_str(int status) {
  switch (status) {
    case SV_OK: return "ok";
    case SV_EINVAL: return "invalid argument";
    case SV_EUNSUPPORTED: return "unsupported";
    case SV_EWORKSPACE: return "workspace too small";
    case SV_EHIP: return "HIP launch failed";
    case SV_ESCRATCH: return "request larger than the static scratch buffer";
    default: return "unknown status";
  }
}

size_t sv_q2_matrix_bytes(int32_t n_out, int32_t k_in) {
  if (n_out < 1 || k_in < 256 || k_in % 256) return 0;
  return q2_bytes((size_t)n_out, (size_t)k_in);
}

size_t sv_q2_tiled_bytes(int32_t n_out, int32_t k_in) {
  if (n_out < 16 || n_out % 16 || k_in < 256 || k_in % 256) return 0;
  return q2_tiled_bytes((size_t)n_out, (size_t)k_in);
}

int sv_q2_tile(const void* src, void* dst, int32_t n_out, int32_t k_in, int32_t parts, int32_t count,
               hipStream_t stream) {
  if (!src || !dst || sv_q2_tiled_bytes(n_out, k_in) == 0 || parts < 1 || parts > 64 || count < 1)
    return SV_EINVAL;
  const size_t nblk = (size_t)count * (size_t)n_out * (size_t)(k_in / 256);
  if (nblk / 256 + 1 > 0x7FFFFFFFu) return SV_EINVAL;   // (grid size)
  const uint8_t *a = (const uint8_t*)src, *b = (const uint8_t*)dst;
  const size_t na = (size_t)count * q2_bytes((size_t)n_out, (size_t)k_in);
  const size_t nbt = (size_t)count * q2_tiled_bytes((size_t)n_out, (size_t)k_in);
  if (a < b + nbt && b < a + na) return SV_EINVAL;   // overlapping buffers
  return hip_status(launch_q2_tile(src, dst, n_out, k_in, parts, count, stream));
}

size_t sv_q8_matrix_bytes(int32_t n_out, int32_t k_in) {
  if (n_out < 1 || k_in < 32 || k_in % 32) return 0;
  return q8_bytes((size_t)n_out, (size_t)k_in);
}

size_t sv_moe_workspace_bytes(const sv_moe_desc* d, int32_t R) {
  if (moe_check(d, R) != SV_OK) return 0;
  return moe_ws_layout(d, R, nullptr, nullptr);
}

int vq2_moe_gemm(const sv_moe_desc* d, const void* x, int32_t x_dtype, int32_t R,
                 const float* router_logits, float* y, int32_t* topk_idx, float* topk_w,
                 void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = moe_check(d, R);
  if (st != SV_OK) return st;
  if (!x || !y || !dtype_ok(x_dtype) || !ws) return SV_EINVAL;
  if (d->ffn == SV_FFN_SWIGLU && d->n_experts > 1 && !router_logits) return SV_EINVAL;
  const size_t need = moe_ws_layout(d, R, nullptr, nullptr);
  if (ws_bytes < need) return SV_EWORKSPACE;
  MoeWs w;
  moe_ws_layout(d, R, ws, &w);
  const bool use_lo = x_dtype == SV_F32;
  if (d->ffn == SV_FFN_PLAIN) {
    st = hip_status(launch_stage(x, x_dtype, R, d->hidden, XL_PERM, nullptr, w.x_img, stream));
    if (st != SV_OK) return st;
    return hip_status(launch_q2_plain(d, R, use_lo, w, y, stream));
  }
  if (!moe_shape_ok(d)) return SV_EUNSUPPORTED;
  st = hip_status(launch_moe_prep(d, R, d->n_experts > 1 ? router_logits : nullptr, x, x_dtype,
                                  topk_idx, topk_w, w, stream));
  if (st != SV_OK) return st;
  st = hip_status(launch_moe_gateup(d, R, w, stream));
  if (st != SV_OK) return st;
  st = hip_status(launch_hdig(d, R, w, stream));
  if (st != SV_OK) return st;
  st = hip_status(launch_moe_down(d, R, w, stream));
  if (st != SV_OK) return st;
  if (shared_q8(d)) {
    plan_shared_q8(d, R, x_dtype, &w);
    st = hip_status(launch_shared_q8(d, R, x, x_dtype, w, stream));
    if (st != SV_OK) return st;
  }
  return hip_status(launch_moe_combine(d, R, w, y, stream));
}

size_t sv_lmhead_workspace_bytes(int32_t hidden, int32_t R) {
  if (hidden < 32 || hidden % 32 || hidden > MAX_K_STAGE || R < 1 || R > SV_MAX_ROWS) return 0;
  return ximg_bytes((size_t)R, (size_t)hidden, XL_PLAIN);
}

int vq8_lmhead_gemm(const void* w, int32_t vocab, int32_t hidden, const void* h,
                    int32_t h_dtype, int32_t R, float* logits, void* ws, size_t ws_bytes,
                    hipStream_t stream) {
  if (!w || !h || !logits || !ws || vocab < 1 || !dtype_ok(h_dtype)) return SV_EINVAL;
  const size_t need = sv_lmhead_workspace_bytes(hidden, R);
  if (need == 0) return SV_EINVAL;
  if (ws_bytes < need) return SV_EWORKSPACE;
  const XImg img = ximg_carve(ws, (size_t)R, hidden, XL_PLAIN);
  int st = hip_status(launch_stage(h, h_dtype, R, hidden, XL_PLAIN, nullptr, img, stream));
  if (st != SV_OK) return st;
  return hip_status(launch_q8_lmhead(w, vocab, hidden, R, h_dtype == SV_F32, img, logits, stream));
}

static bool accept_shape_ok(int32_t S, int32_t K, int32_t V) {
  if (S < 1 || K < 0 || K > SV_MAX_DRAFTS || V < 1 || V > 256 * 2048) return false;
  return (long long)S * (2 * K + 1) <= 65535;
}

size_t sv_accept_workspace_bytes(int32_t S, int32_t K, int32_t V) {
  if (!accept_shape_ok(S, K, V)) return 0;
  return accept_ws_bytes(S, K, V);
}

// Target-sample matching launches one block row per target row only.
static bool tsm_shape_ok(int32_t S, int32_t K, int32_t V) {
  if (S < 1 || K < 0 || K > SV_MAX_DRAFTS || V < 1 || V > 256 * 2048) return false;
  return (long long)S * (K + 1) <= 65535;
}

size_t sv_accept_tsm_workspace_bytes(int32_t S, int32_t K, int32_t V) {
  if (!tsm_shape_ok(S, K, V)) return 0;
  return accept_tsm_ws_bytes(S, K, V);
}

int spec_accept_target_sample(int32_t S, int32_t K, int32_t V, const float* target,
                              int32_t target_kind, float T_p, const int32_t* draft_tokens,
                              const float* uniforms, int32_t* out_tokens, int32_t* out_n_accepted,
                              void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!tsm_shape_ok(S, K, V)) return SV_EINVAL;
  if (!target || !uniforms || !out_tokens || !out_n_accepted || !ws) return SV_EINVAL;
  if (K > 0 && !draft_tokens) return SV_EINVAL;
  if (!kind_ok(target_kind)) return SV_EINVAL;
  if (target_kind == SV_LOGITS && !(isfinite(T_p) && T_p >= 0.f)) return SV_EINVAL;
  if (ws_bytes < accept_tsm_ws_bytes(S, K, V)) return SV_EWORKSPACE;
  return hip_status(launch_accept_tsm(S, K, V, target, target_kind, T_p, draft_tokens, uniforms,
                                      out_tokens, out_n_accepted, ws, stream));
}

int sv_spec_account(const int32_t* n_accepted, int32_t S, int32_t K, double guard, double threshold,
                    sv_spec_account_t* state) {
  if (!n_accepted || !state || S < 1 || K < 0 || K > SV_MAX_DRAFTS) return SV_EINVAL;
  if (!isfinite(guard) || !isfinite(threshold)) return SV_EINVAL;
  for (int32_t s = 0; s < S; ++s)
    if (n_accepted[s] < -1 || n_accepted[s] > K) return SV_EINVAL;
  for (int32_t s = 0; s < S; ++s) {
    sv_spec_account_t& a = state[s];
    if (a.quenched || n_accepted[s] < 0) continue;
    const int64_t t = (int64_t)n_accepted[s] + 1;
    a.steps += 1;
    a.tokens += t;
    a.regret += guard - (double)t;
    if (a.regret > threshold) {
      a.quenched = 1;
      a.quench_step = (int32_t)a.steps;
    }
  }
  return SV_OK;
}

}  // extern "C"

// Scratch memory of spec_accept_noalloc: one copy per GPU, for the life of the
// process.  In host code `scratch` only names the symbol; its device address
// (different on every GPU) comes from hipGetSymbolAddress, looked up once per
// device on that device's first call and cached.
static __device__ __align__(256) uint8_t scratch[SV_ACCEPT_SCRATCH_BYTES];

namespace {

int accept_args_ok(int32_t S, int32_t K, int32_t V, const float* target, int32_t target_kind,
                   float T_p, const float* draft, int32_t draft_kind, float T_q,
                   const int32_t* draft_tokens, const float* uniforms, int32_t* out_tokens,
                   int32_t* out_n_accepted) {
  if (!accept_shape_ok(S, K, V)) return SV_EINVAL;
  if (!target || !uniforms || !out_tokens || !out_n_accepted) return SV_EINVAL;
  if (K > 0 && (!draft || !draft_tokens)) return SV_EINVAL;
  if (!kind_ok(target_kind) || (K > 0 && !kind_ok(draft_kind))) return SV_EINVAL;
  if (target_kind == SV_LOGITS && !(isfinite(T_p) && T_p >= 0.f)) return SV_EINVAL;
  if (K > 0 && draft_kind == SV_LOGITS && !(isfinite(T_q) && T_q >= 0.f)) return SV_EINVAL;
  return SV_OK;
}

constexpr int MAX_DEV = 64;
std::atomic<void*> scratch_ptr[MAX_DEV];

// Device address of this device's scratch array, or null (lookup failed).
void* scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEV) return nullptr;
  void* p = scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
  scratch_ptr[dev].store(p, std::memory_order_release);
  return p;
}

}  // namespace

extern "C" {

int spec_accept(int32_t S, int32_t K, int32_t V, const float* target, int32_t target_kind,
                float T_p, const float* draft, int32_t draft_kind, float T_q,
                const int32_t* draft_tokens, const float* uniforms, int32_t* out_tokens,
                int32_t* out_n_accepted, void* ws, size_t ws_bytes, hipStream_t stream) {
  const int st = accept_args_ok(S, K, V, target, target_kind, T_p, draft, draft_kind, T_q,
                                draft_tokens, uniforms, out_tokens, out_n_accepted);
  if (st != SV_OK) return st;
  if (!ws) return SV_EINVAL;
  if (ws_bytes < accept_ws_bytes(S, K, V)) return SV_EWORKSPACE;
  return hip_status(launch_accept(S, K, V, target, target_kind, T_p, draft,
                                  K > 0 ? draft_kind : target_kind, T_q, draft_tokens, uniforms,
                                  out_tokens, out_n_accepted, ws, stream));
}

int spec_accept_noalloc(int32_t S, int32_t K, int32_t V, const float* target, int32_t target_kind,
                        float T_p, const float* draft, int32_t draft_kind, float T_q,
                        const int32_t* draft_tokens, const float* uniforms, int32_t* out_tokens,
                        int32_t* out_n_accepted, hipStream_t stream) {
  const int st = accept_args_ok(S, K, V, target, target_kind, T_p, draft, draft_kind, T_q,
                                draft_tokens, uniforms, out_tokens, out_n_accepted);
  if (st != SV_OK) return st;
  if (accept_ws_bytes(S, K, V) > SV_ACCEPT_SCRATCH_BYTES) return SV_ESCRATCH;
  void* ws = scratch_address();
  if (!ws) return SV_EHIP;
  // the same kernels as spec_accept, on the scratch array; the per-sequence
  // counters they need at zero are cleared by the first of them
  return hip_status(launch_accept(S, K, V, target, target_kind, T_p, draft,
                                  K > 0 ? draft_kind : target_kind, T_q, draft_tokens, uniforms,
                                  out_tokens, out_n_accepted, ws, stream));
}

int vq2_dequant(const void* w, int32_t n_out, int32_t k_in, float* out, hipStream_t stream) {
  if (!w || !out || sv_q2_matrix_bytes(n_out, k_in) == 0) return SV_EINVAL;
  return hip_status(launch_q2_dequant(w, n_out, k_in, out, stream));
}

int sv_read_probe(const void* src, size_t bytes, int32_t mode, uint32_t* sink, size_t sink_words,
                  hipStream_t stream) {
  if (!src || !sink || mode < 0 || mode > 5 || bytes < SV_PROBE_GROUP_BYTES) return SV_EINVAL;
  if (sink_words < read_probe_sink_words()) return SV_EWORKSPACE;
  return hip_status(launch_read_probe(src, bytes, mode, sink, stream));
}

int vq8_dequant(const void* w, int32_t n_out, int32_t k_in, float* out, hipStream_t stream) {
  if (!w || !out || sv_q8_matrix_bytes(n_out, k_in) == 0) return SV_EINVAL;
  return hip_status(launch_q8_dequant(w, n_out, k_in, out, stream));
}

}  // extern "C"

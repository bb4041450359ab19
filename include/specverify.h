/*
 * libspecverify -- the target-model verifier step of lossless speculative
 * decoding over a two-bit mixture-of-experts model, as hand-written HIP kernels
 * for AMD MI355X (gfx950).
 *
 * Sources (web pages; cited by title and section):
 *  [T1] "Optimizing DeepSeek-V4-Flash on a single NVIDIA GB10/GX10 with DSpark
 *       speculative decoding", forum thread, page 1 (post 1: the p/q rule,
 *       the verifier as the bottleneck; post 20: per-session RNG and state in
 *       multi-session cohorts) and page 2 (the author's verifier post: K+1
 *       rows through routed MoE, projections and the vocabulary head).
 *  [T3] "ds4-on-spark" README (introduction: block formats of the weights,
 *       expert dedup; "Roofline": decode is weight-streaming bound; "Under the
 *       hood": routed experts stay quantised with inline dequantisation; "The
 *       break-even law": one committed row plus four draft rows per verify,
 *       the break-even guard and the yield-quench controller).
 *  [T4] "1x Spark tuned DSpark for DeepSeek-V4-Flash: 35 tok/s, 800+ prefill,
 *       and fast multi-agent serving", forum thread (Q&A answer 3: fused
 *       gate+up+SwiGLU MoE decode, fused router; "The break-even law, and why
 *       speculation can't hurt you here": the realised regret per verify step,
 *       and the verify rows as the only token source).
 *
 * Conventions for every call:
 *  - Pointers are DEVICE pointers unless marked (host).  The caller owns all
 *    memory, including workspaces; the library never allocates, frees or
 *    synchronises.  Its only global state: a per-device cache of the
 *    compute-unit count (used to size persistent grids), and the static scratch
 *    array of spec_accept_noalloc with its per-device address.
 *  - Work is enqueued on `stream` (0 = the null stream).  Calls on different
 *    streams are independent when their workspaces and outputs are distinct.
 *  - Arguments are validated on the host before anything is enqueued; a
 *    failure returns SV_EINVAL (or SV_EWORKSPACE) and changes nothing.  A
 *    failed launch returns SV_EHIP.  Bad *device data* (e.g. a draft token out
 *    of range) cannot be reported synchronously; spec_accept marks the affected
 *    sequence with -1 outputs instead.  No kernel traps.
 *  - Row-major layouts throughout.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;

#if defined(__GNUC__)
#define SV_API __attribute__((visibility("default")))
#else
#define SV_API
#endif

enum sv_status {
  SV_OK = 0,
  SV_EINVAL = 1,        /* invalid argument; nothing enqueued */
  SV_EUNSUPPORTED = 2,  /* valid but outside what the library implements */
  SV_EWORKSPACE = 3,    /* workspace smaller than the matching *_workspace_bytes() */
  SV_EHIP = 4,          /* a HIP launch failed */
  SV_ESCRATCH = 5       /* needs more than the library's static scratch buffer */
};

enum sv_dtype { SV_F32 = 0, SV_BF16 = 1 };   /* element type of activation rows */

enum sv_ffn {
  SV_FFN_PLAIN = 0,   /* y = W x with W = w_gate [inter x hidden]; n_experts = top_k = 1 */
  SV_FFN_SWIGLU = 1   /* y = W_d (silu(W_g x) * (W_u x)) per expert, routed + optional shared */
};

enum sv_dist { SV_LOGITS = 0, SV_PROBS = 1 };  /* how a distribution row is given */

enum sv_wfmt { SV_Q2 = 0, SV_Q8 = 1 };         /* block format of the shared expert */

#define SV_API_VERSION 3
#define SV_MAX_ROWS 64        /* R limit of the GEMM calls */
#define SV_MAX_TOPK 16
#define SV_MAX_EXPERTS 1024
#define SV_MAX_DRAFTS 31      /* K limit of spec_accept */

SV_API int sv_api_version(void);
SV_API const char* sv_status_str(int status);

/*
 * Two-bit block matrix ("Q2_K" is named for routed-expert weights in [T3],
 * introduction; the pages give no bit layout -- this is the library's own).
 * [n_out x k_in], k_in % 256 == 0; nb = k_in/256 blocks per output row; block
 * index b = n*nb + kb.  Four planes, each at a 256-byte-aligned offset from the
 * start of the matrix:
 *   codes   nblk*64 B : element e of block b = (codes[64b + e/4] >> 2*(e%4)) & 3
 *   nibbles nblk*16 B : byte j <-> elements 16j..16j+15; low nibble scale sc,
 *                       high nibble min m
 *   d       nblk fp16 : block scale
 *   dmin    nblk fp16 : block min-scale
 * weight = d*sc*q - dmin*m.  Returns the matrix size in bytes (sum of the
 * 256-aligned plane sizes), or 0 for invalid shapes.  Matrices of one tensor
 * (e.g. all experts' gate matrices) are stored back to back, each this long.
 */
SV_API size_t sv_q2_matrix_bytes(int32_t n_out, int32_t k_in);

/*
 * Expert-tiled two-bit matrix: the blocks of a two-bit matrix regrouped so
 * that everything one step of the SwiGLU expert kernels reads -- codes,
 * nibbles, d and dmin of one or two blocks of 16 consecutive output rows --
 * is one contiguous chunk (whole 128-byte lines instead of pieces of four
 * planes).  The layout is the library's own (decode is bound by streaming the
 * weights: [T3] "Roofline"); values and block format are unchanged.
 * n_out % 16 == 0, k_in % 256 == 0, nb = k_in/256.  `parts` is the number of
 * K ranges the kernels split a row into (4 for gate and up, 1 for down): part
 * p covers blocks [nb*p/parts, nb*(p+1)/parts) (integer division).  A part's
 * blocks form steps: one block first when the part starts at an odd block,
 * then aligned pairs (2k, 2k+1), then one block when one is left.  The step of
 * tile t (rows 16t .. 16t+15) starting at block kb with nblk blocks is the
 * chunk of 1344*nblk bytes at byte 1344*(t*nb + kb):
 *   codes   [16 rows][64*nblk B]: 16-byte piece c of row r (bytes 16c ..
 *           16c+15 of its nblk*64 code bytes) at r*64*nblk + 16*((c+r) mod 4*nblk)
 *   nibbles [nblk][4][16 rows] dwords from byte 1024*nblk: dword g (nibble
 *           bytes 4g .. 4g+3) of block j of the step, row r, at
 *           1024*nblk + 4*(16*(4j + g) + r)
 *   d       [16 rows][nblk] fp16 from byte 1280*nblk
 *   dmin    [16 rows][nblk] fp16 from byte 1312*nblk
 * sv_q2_tiled_bytes returns the size (84 bytes per 256 weights, no padding) or
 * 0 for invalid shapes.
 */
SV_API size_t sv_q2_tiled_bytes(int32_t n_out, int32_t k_in);

/*
 * Regroups `count` two-bit matrices [n_out x k_in] stored back to back in the
 * layout above (src, each sv_q2_matrix_bytes long) into the expert-tiled
 * layout (dst, each sv_q2_tiled_bytes long), on `stream`.  src and dst are
 * device buffers that must not overlap; the call only enqueues the copy.
 * Returns SV_EINVAL for invalid shapes, parts outside 1..64, count < 1 or null
 * pointers.
 */
SV_API int sv_q2_tile(const void* src, void* dst, int32_t n_out, int32_t k_in, int32_t parts, int32_t count,
                      hipStream_t stream);

/*
 * Eight-bit block matrix ("Q8_0" for the output head in [T3], introduction):
 * [n_out x k_in], k_in % 32 == 0; blocks of 32 int8 codes with one fp16 scale;
 * block b = n*(k_in/32) + kb.  Planes: codes nblk*32 int8, then d nblk fp16,
 * each 256-byte aligned.  weight = d*q.  Returns the size in bytes, or 0.
 */
SV_API size_t sv_q8_matrix_bytes(int32_t n_out, int32_t k_in);

/*
 * Description of one MoE layer (host struct, read only during the call).
 *  SV_FFN_SWIGLU: w_gate, w_up: n_experts matrices [inter x hidden] each,
 *    expert-tiled with parts = 4 (sv_q2_tile), back to back
 *    sv_q2_tiled_bytes(inter, hidden) apart; w_down: n_experts matrices
 *    [hidden x inter], expert-tiled with parts = 1; s_gate/s_up/s_down: the
 *    shared expert (always on, combine weight 1) or all NULL.  s_format
 *    SV_Q2: the shared matrices in the routed experts' layouts; SV_Q8: the
 *    shared matrices eight-bit (the format the pages' model keeps its shared
 *    expert in: [T3] introduction, the quantisation recipe; [T1] page 1, post
 *    14, the target file's name), s_gate/s_up [inter x hidden] and s_down
 *    [hidden x inter] in the plain eight-bit layout below, each computed with
 *    the vocabulary head's kernels (activation rows staged as fp16 high +
 *    remainder).  Ignored when there is no shared expert.
 *  SV_FFN_PLAIN: w_gate is one [inter x hidden] two-bit matrix (plain
 *    layout); the other five NULL; n_experts = top_k = 1.
 *  hidden % 256 == 0 and inter % 256 == 0 for SWIGLU; PLAIN needs
 *  hidden % 256 == 0 and inter >= 1.
 */
typedef struct {
  int32_t ffn, hidden, inter, n_experts, top_k;
  const void *w_gate, *w_up, *w_down;
  const void *s_gate, *s_up, *s_down;
  int32_t s_format;   /* sv_wfmt of s_gate / s_up / s_down */
} sv_moe_desc;

/* Workspace bytes vq2_moe_gemm needs for this layer and R rows (0 if invalid). */
SV_API size_t sv_moe_workspace_bytes(const sv_moe_desc* d, int32_t R);

/*
 * Routed two-bit MoE layer for R verifier rows (steps: activation staging,
 * router top-k, expert grouping with dedup ([T3] introduction, "MoE gate_up
 * expert dedup"), fused gate+up+SwiGLU ([T4] Q&A 3), down projection and the
 * weighted combine).  Weights stay quantised in HBM and are dequantised in
 * registers ([T3] "Under the hood"); each weight tile is read once for all rows
 * routed to its expert.
 *
 *  x             [R, hidden], x_dtype SV_F32 or SV_BF16; 1 <= R <= SV_MAX_ROWS
 *  router_logits [R, n_experts] fp32; may be NULL only when n_experts == 1
 *  y             [R, hidden] fp32 (PLAIN: [R, inter])
 *  topk_idx      [R, top_k] int32 output or NULL: the top_k experts by router
 *                logit, largest first, ties to the lower index
 *  topk_w        [R, top_k] fp32 output or NULL: softmax probability of each
 *                chosen expert over all n_experts (not renormalised)
 *  ws, ws_bytes  device workspace of at least sv_moe_workspace_bytes(d, R)
 *
 *  y_r = sum_s topk_w[r,s] * FFN_{topk_idx[r,s]}(x_r) + FFN_shared(x_r), with
 *  FFN(x) = W_d(silu(W_g x) * (W_u x)) and fp32 intermediates.  Summation
 *  order is fixed, so results are run-to-run deterministic.  Accuracy: every
 *  element of y within 2e-3 relative of the exact value, or of 1e-3 of its
 *  row's largest magnitude where that is larger (x and h enter the two-bit
 *  products as ~30-bit fixed-point values per row, exact for bf16 x within
 *  2^-22 of the row's largest magnitude; the eight-bit shared expert takes
 *  its rows as fp16 high + remainder, ~22 significant bits).
 */
SV_API int vq2_moe_gemm(const sv_moe_desc* d, const void* x, int32_t x_dtype, int32_t R,
                 const float* router_logits, float* y, int32_t* topk_idx, float* topk_w,
                 void* ws, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes vq8_lmhead_gemm needs (0 if invalid). */
SV_API size_t sv_lmhead_workspace_bytes(int32_t hidden, int32_t R);

/*
 * Vocabulary head in eight-bit blocks: logits[r, v] = sum_k W[v, k] h[r, k],
 * W an eight-bit matrix [vocab x hidden] (hidden % 32 == 0), h [R, hidden] in
 * h_dtype, logits [R, vocab] fp32.  Each weight tile is read once and reused
 * for all R rows (the "Q8 tiny-batch reuse" of [T1] post 1).
 */
SV_API int vq8_lmhead_gemm(const void* w, int32_t vocab, int32_t hidden, const void* h,
                    int32_t h_dtype, int32_t R, float* logits, void* ws, size_t ws_bytes,
                    hipStream_t stream);

/* Workspace bytes spec_accept needs (0 if invalid). */
SV_API size_t sv_accept_workspace_bytes(int32_t S, int32_t K, int32_t V);

/*
 * The p/q accept/reject rule with residual resampling ([T1] post 1: drafts are
 * sampled from q, the target defines p, accept with probability
 * min(1, p(x)/q(x)), a rejected draft is replaced from the normalised positive
 * residual max(0, p - q)), for S independent sequences of K drafts each
 * (cohorts with per-session state: [T1] post 20).
 *
 *  target        [S*(K+1), V] fp32; row s*(K+1)+i is position i of sequence s
 *                (the K+1 verifier rows: [T1] page 2; [T3] "The break-even law")
 *  target_kind   SV_LOGITS: p = softmax(row / T_p), or for T_p == 0 (greedy
 *                decoding: [T1] page 1, post 12; [T4] Q&A, the FP8 KV answer,
 *                the self-check at temperature 0) the one-hot distribution at
 *                the row's first largest value; SV_PROBS: p = row as given
 *  draft         [S*K, V] fp32, row s*K+i; q likewise with draft_kind / T_q;
 *                may be NULL when K == 0
 *  draft_tokens  [S, K] int32
 *  uniforms      [S, K+1] fp32 in [0, 1): u[s][i] decides draft i, u[s][K]
 *                drives the one inverse-CDF sample
 *  out_tokens    [S, K+1] int32: the n accepted drafts, then the correction
 *                token (on a rejection) or the bonus token from row K (when all
 *                K pass), then -1 padding
 *  out_n_accepted [S] int32
 *
 *  Per sequence, for i = 0..K-1: accept iff u_i*q_i(d_i) < p_i(d_i), evaluated
 *  exactly; on the first reject emit the first x (vocabulary order) whose
 *  running sum of r = max(0, p_i - q_i) exceeds u_K * sum(r) (if sum(r) == 0,
 *  sample p_i the same way) and stop; if all pass, sample p_K the same way.
 *  Distributions are evaluated in fp64.  A sequence with a draft token outside
 *  [0, V), a uniform outside [0, 1), a non-finite value, or (SV_PROBS) a
 *  negative value or an all-zero row gets -1 in every output slot.
 *  T_p / T_q must be finite and >= 0 for SV_LOGITS rows (0: greedy; then the
 *  output is the longest prefix of drafts equal to their rows' largest target
 *  logits, followed by the largest logit of the next row).  1 <= S, 0 <= K <=
 *  SV_MAX_DRAFTS, 1 <= V <= 524,288, S (2K+1) <= 65,535.
 */
SV_API int spec_accept(int32_t S, int32_t K, int32_t V, const float* target, int32_t target_kind,
                float T_p, const float* draft, int32_t draft_kind, float T_q,
                const int32_t* draft_tokens, const float* uniforms, int32_t* out_tokens,
                int32_t* out_n_accepted, void* ws, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes spec_accept_target_sample needs (0 if invalid). */
SV_API size_t sv_accept_tsm_workspace_bytes(int32_t S, int32_t K, int32_t V);

/*
 * Target-sample matching ([T4] "The break-even law, and why speculation can't
 * hurt you here", the paragraph on losslessness: the verify forward is the only
 * token source; the accept loop draws the target's own token from each verify
 * row with the request's sampler and random stream).  For S sequences of K
 * drafts: t_i = the first x (vocabulary order) whose running sum of p_i
 * exceeds u[s][i] times the row total, for every row i = 0..K; n = the first
 * i < K with t_i != draft i (K if none); the outputs are drafts 0..n-1, then
 * t_n, then -1 padding.  No draft distribution is read.  target,
 * target_kind, T_p, draft_tokens, uniforms ([S, K+1]: u[s][i] samples row i),
 * out_tokens, out_n_accepted, validation, and the -1 marking of sequences with
 * invalid data are as for spec_accept; draft_tokens may be NULL when K == 0.
 * With T_p == 0 (greedy rows) the output equals spec_accept's.  1 <= S,
 * 0 <= K <= SV_MAX_DRAFTS, 1 <= V <= 524,288, S (K+1) <= 65,535.
 */
SV_API int spec_accept_target_sample(int32_t S, int32_t K, int32_t V, const float* target,
                int32_t target_kind, float T_p, const int32_t* draft_tokens,
                const float* uniforms, int32_t* out_tokens, int32_t* out_n_accepted,
                void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Step accounting of the yield-quench policy ([T3] "The break-even law": a
 * verify step costs about `guard` plain decode steps, so it pays only when it
 * commits more tokens than that; the controller sums guard - tokens per step
 * and turns speculation off for the rest of the request once the sum exceeds a
 * few plain-step times; [T4] "The break-even law, and why speculation can't
 * hurt you here": the realised regret guard - tokens committed, summed per
 * verify step, a terminal quench).  A HOST function over one verify step's
 * out_n_accepted, copied to host memory.
 *
 *  n_accepted  [S] (host) int32, as an accept call wrote it: -1 marks a
 *              sequence whose inputs were invalid (nothing committed; the step
 *              is not counted); otherwise 0..K
 *  state       [S] (host), in/out; zero-initialised before a request's first
 *              step
 *
 * For each sequence not yet quenched with n >= 0: t = n + 1 tokens
 * committed; steps += 1; tokens += t; regret += guard - t (fp64, not clamped
 * at zero, so early gains are banked); if regret > threshold: quenched = 1,
 * quench_step = steps.  Quenched sequences are left as they are.  SV_EINVAL,
 * with no state changed, for null pointers, S < 1, K outside 0..SV_MAX_DRAFTS,
 * an n outside -1..K, or a non-finite guard or threshold.
 */
typedef struct {
  int64_t steps;         /* verify steps counted */
  int64_t tokens;        /* tokens committed by them */
  double regret;         /* sum of guard - tokens committed */
  int32_t quenched;      /* 1 once regret exceeded the threshold */
  int32_t quench_step;   /* the step at which it did (0 while not quenched) */
} sv_spec_account_t;
SV_API int sv_spec_account(const int32_t* n_accepted, int32_t S, int32_t K, double guard,
                           double threshold, sv_spec_account_t* state);

/*
 * spec_accept without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments, rule, outputs and validation as
 * spec_accept; its scratch memory is a static device array of
 * SV_ACCEPT_SCRATCH_BYTES inside the library (one per GPU, held until the
 * process ends; its address is looked up on the first call on each device).
 * Allocates nothing.  Returns SV_ESCRATCH, with nothing enqueued, when
 * sv_accept_workspace_bytes(S, K, V) exceeds SV_ACCEPT_SCRATCH_BYTES (at
 * V = 129,280 and K = 4: up to 31 sequences).  Every call on one GPU uses that
 * GPU's one array: calls whose executions overlap on one GPU (different
 * streams, or several host threads) race and give undefined results; calls
 * ordered on one stream are safe.
 */
#define SV_ACCEPT_SCRATCH_BYTES ((size_t)16 << 20)
SV_API int spec_accept_noalloc(int32_t S, int32_t K, int32_t V, const float* target,
                int32_t target_kind, float T_p, const float* draft, int32_t draft_kind,
                float T_q, const int32_t* draft_tokens, const float* uniforms,
                int32_t* out_tokens, int32_t* out_n_accepted, hipStream_t stream);

/*
 * Test exports: the dequantised weights [n_out, k_in] fp32.  Two-bit: the exact
 * value d*sc*q - dmin*m rounded once to fp32 (nearest, ties to even);
 * eight-bit: d*q (exact).
 */
SV_API int vq2_dequant(const void* w, int32_t n_out, int32_t k_in, float* out, hipStream_t stream);
SV_API int vq8_dequant(const void* w, int32_t n_out, int32_t k_in, float* out, hipStream_t stream);

/*
 * Tooling: a read-bandwidth probe, the measured denominator of the roofline
 * fractions ([T3] "Roofline": a bandwidth probe sets the achievable rate).
 * Reads floor(bytes / SV_PROBE_GROUP_BYTES) groups of 16 rows x 1792 bytes
 * (the code plane of a 16-row tile of a 7168-wide two-bit matrix) from `src`
 * once, each wave a contiguous range, 1 KB per wave instruction, in pattern
 * `mode`: 0 loads into registers over full 128-byte lines; 1 global-to-LDS
 * loads, non-temporal, full lines; 2 the same with the default cache policy;
 * 3 global-to-LDS loads in 64-byte pieces (16 rows x 64 B per instruction);
 * 4 the same, non-temporal; 5 global-to-LDS 4-byte loads, non-temporal, 256
 * contiguous bytes per instruction (the first 7 KB of every group only).
 * `sink` [sink_words] receives one word per wave (at most 8 per compute
 * unit); SV_EWORKSPACE if sink_words is smaller.
 */
#define SV_PROBE_GROUP_BYTES ((size_t)16 * 1792)
SV_API int sv_read_probe(const void* src, size_t bytes, int32_t mode, uint32_t* sink,
                         size_t sink_words, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */

// Internal declarations shared by the HIP translation units of libspecverify.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "specverify.h"

namespace sv {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));

__host__ __device__ inline size_t up256(size_t n) { return (n + 255) & ~size_t(255); }

// Index of the calling wave in its block, as a wave-uniform (scalar) value:
// the compiler cannot tell that threadIdx.x / 64 is uniform, and everything
// derived from it would otherwise be computed per lane.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Block barrier after this wave's LDS writes are done, leaving its vector
// memory loads in flight (the LDS-scope part of __syncthreads only).
__device__ __forceinline__ void barrier_lds() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt at their maxima
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ------------------------------------------------------ cross-lane moves
// Wave-wide reductions on the VALU: DPP moves inside 16-lane rows and the
// permlane16/permlane32 swaps across rows, instead of LDS permutes.
// xlane<CTRL>(x): lane i takes x from another lane under the DPP control
// CTRL: 0xB1 quad_perm [1,0,3,2], 0x4E quad_perm [2,3,0,1], 0x141
// row_half_mirror, 0x140 row_mirror.
template <int CTRL>
__device__ __forceinline__ uint32_t xlane(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ double xlane(double x) {
  const uint64_t b = __builtin_bit_cast(uint64_t, x);
  const uint64_t lo = xlane<CTRL>((uint32_t)b), hi = xlane<CTRL>((uint32_t)(b >> 32));
  return __builtin_bit_cast(double, lo | (hi << 32));
}
template <int CTRL>
__device__ __forceinline__ float xlane(float x) {
  return __builtin_bit_cast(float, xlane<CTRL>(__builtin_bit_cast(uint32_t, x)));
}

// The permlane swaps pair the even and odd 16-lane rows (SPAN 16) or the two
// 32-lane halves (SPAN 32): every lane gets (even / low part, odd / high
// part) of its pair, so op(a, b) is the same expression in all lanes.
template <int SPAN>
__device__ __forceinline__ void xswap(uint32_t x, uint32_t& a, uint32_t& b) {
  const auto r = SPAN == 16 ? __builtin_amdgcn_permlane16_swap(x, x, false, false)
                            : __builtin_amdgcn_permlane32_swap(x, x, false, false);
  a = r[0];
  b = r[1];
}
template <int SPAN>
__device__ __forceinline__ void xswap(double x, double& a, double& b) {
  const uint64_t v = __builtin_bit_cast(uint64_t, x);
  uint32_t la, lb, ha, hb;
  xswap<SPAN>((uint32_t)v, la, lb);
  xswap<SPAN>((uint32_t)(v >> 32), ha, hb);
  a = __builtin_bit_cast(double, (uint64_t)la | ((uint64_t)ha << 32));
  b = __builtin_bit_cast(double, (uint64_t)lb | ((uint64_t)hb << 32));
}
template <int SPAN>
__device__ __forceinline__ void xswap(float x, float& a, float& b) {
  uint32_t ua, ub;
  xswap<SPAN>(__builtin_bit_cast(uint32_t, x), ua, ub);
  a = __builtin_bit_cast(float, ua);
  b = __builtin_bit_cast(float, ub);
}

// op over the 64 lanes, the result in every lane (bit-identical in all
// lanes and in every wave: a fixed pairing, commutative op).
template <typename T, typename Op>
__device__ __forceinline__ T wave_allreduce(T v, Op op) {
  v = op(v, xlane<0xB1>(v));
  v = op(v, xlane<0x4E>(v));
  v = op(v, xlane<0x141>(v));
  v = op(v, xlane<0x140>(v));
  T a, b;
  xswap<16>(v, a, b);
  v = op(a, b);
  xswap<32>(v, a, b);
  return op(a, b);
}

// op over each 32-lane half of the wave, the result in every lane of the half
// (the same pairing in every half: bit-identical there).
template <typename T, typename Op>
__device__ __forceinline__ T half_allreduce(T v, Op op) {
  v = op(v, xlane<0xB1>(v));
  v = op(v, xlane<0x4E>(v));
  v = op(v, xlane<0x141>(v));
  v = op(v, xlane<0x140>(v));
  T a, b;
  xswap<16>(v, a, b);
  return op(a, b);
}

// Sum over the lanes l, l ^ 16, l ^ 32, l ^ 48 (the four 16-lane rows), in
// every lane: (x0 + x1) + (x2 + x3).
__device__ __forceinline__ float rows_sum(float v) {
  float a, b;
  xswap<16>(v, a, b);
  v = a + b;
  xswap<32>(v, a, b);
  return a + b;
}

// s_waitcnt that waits until at most n vector-memory loads are outstanding
// (n a compile-time constant after inlining), leaving the other counters alone.
__device__ __forceinline__ void wait_vmcnt_le(int n) {
  asm volatile("" ::: "memory");   // no later load may be hoisted above the wait
#define SV_W(N) case N: __builtin_amdgcn_s_waitcnt(((N) & 0xF) | ((((N) >> 4) & 3) << 14) | (0x7 << 4) | (0xF << 8)); break;
  switch (n) {
    SV_W(0) SV_W(1) SV_W(2) SV_W(3) SV_W(4) SV_W(5) SV_W(6) SV_W(7) SV_W(8) SV_W(9)
    SV_W(10) SV_W(11) SV_W(12) SV_W(13) SV_W(14) SV_W(15) SV_W(16) SV_W(17) SV_W(18)
    SV_W(19) SV_W(20) SV_W(21) SV_W(22) SV_W(23) SV_W(24) SV_W(25) SV_W(26) SV_W(27)
    SV_W(28) SV_W(29) SV_W(30) SV_W(31)
    default: __builtin_amdgcn_s_waitcnt(0); break;   // (more loads than encodable: wait for all)
  }
#undef SV_W
}

// silu(g) * u in fp32 (the SwiGLU of the expert layers).
__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.f + expf(-g)) * u; }

// ---------------------------------------------------- global-to-LDS loads
// One wave instruction: lane l copies 4 or 16 bytes from its own global
// address `src` to LDS byte address la + 4 l or la + 16 l (la wave-uniform).
// Written as inline assembly because the compiler, seeing such a load
// outstanding, would wait for every vector load before the next use; callers
// wait with explicit vmcnt counts instead.  nt: the non-temporal hint, for
// data read exactly once (full 128-byte lines stream fastest with it).
__device__ __forceinline__ void dma16(const void* src, uint32_t la) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(src), "s"(__builtin_amdgcn_readfirstlane(la)) : "memory", "m0");
}
__device__ __forceinline__ void dma16_nt(const void* src, uint32_t la) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt"
               :: "v"(src), "s"(__builtin_amdgcn_readfirstlane(la)) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* src, uint32_t la) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off"
               :: "v"(src), "s"(__builtin_amdgcn_readfirstlane(la)) : "memory", "m0");
}

// The same with a wave-uniform base address in scalar registers and a 32-bit
// per-lane byte offset (the address is base + off): a loop that streams a
// fixed per-lane pattern moves only the scalar base.
__device__ __forceinline__ void dma16s(const void* base, uint32_t off, uint32_t la) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(off), "s"(base), "s"(__builtin_amdgcn_readfirstlane(la)) : "memory", "m0");
}
__device__ __forceinline__ void dma16s_nt(const void* base, uint32_t off, uint32_t la) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt"
               :: "v"(off), "s"(base), "s"(__builtin_amdgcn_readfirstlane(la)) : "memory", "m0");
}
__device__ __forceinline__ void dma4s(const void* base, uint32_t off, uint32_t la) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1"
               :: "v"(off), "s"(base), "s"(__builtin_amdgcn_readfirstlane(la)) : "memory", "m0");
}

// LDS byte address of a generic pointer into the LDS aperture.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}

// A global pointer to data that no kernel of this launch writes, in the
// constant address space: uniform reads through it become scalar loads even
// in kernels that store to global memory (the compiler cannot otherwise rule
// out that the stores change the data).
template <typename T>
__device__ __forceinline__ const __attribute__((address_space(4))) T* const_ptr(const T* p) {
  return (const __attribute__((address_space(4))) T*)p;
}

// ---------------------------------------------------------------- formats
// Two-bit matrix [n_out x k_in]: planes codes / nibbles / d / dmin, each at a
// 256-byte aligned offset (layout documented in specverify.h).
struct Q2View {
  const uint8_t* qs;   // nblk*64
  const uint8_t* sc;   // nblk*16
  const uint16_t* d;   // nblk fp16 bits
  const uint16_t* dm;  // nblk fp16 bits
  int nb;              // blocks per output row = k_in / 256
  int n_out;
};

__host__ __device__ inline size_t q2_bytes(size_t n_out, size_t k_in) {
  size_t nblk = n_out * (k_in / 256);
  return up256(nblk * 64) + up256(nblk * 16) + 2 * up256(nblk * 2);
}

// Expert-tiled two-bit matrix (sv_q2_tile): 84 bytes per 256 weights.
__host__ __device__ inline size_t q2_tiled_bytes(size_t n_out, size_t k_in) { return n_out * (k_in / 256) * 84; }

__host__ __device__ inline Q2View q2_view(const void* base, int n_out, int k_in) {
  const uint8_t* p = (const uint8_t*)base;
  size_t nblk = (size_t)n_out * (k_in / 256);
  Q2View v;
  v.qs = p;
  v.sc = p + up256(nblk * 64);
  v.d = (const uint16_t*)(v.sc + up256(nblk * 16));
  v.dm = (const uint16_t*)((const uint8_t*)v.d + up256(nblk * 2));
  v.nb = k_in / 256;
  v.n_out = n_out;
  return v;
}

// Eight-bit matrix: codes nblk*32 int8, then d nblk fp16.
struct Q8View {
  const int8_t* qs;
  const uint16_t* d;
  int nb;  // k_in / 32
  int n_out;
};

__host__ __device__ inline size_t q8_bytes(size_t n_out, size_t k_in) {
  size_t nblk = n_out * (k_in / 32);
  return up256(nblk * 32) + up256(nblk * 2);
}

__host__ __device__ inline Q8View q8_view(const void* base, int n_out, int k_in) {
  const uint8_t* p = (const uint8_t*)base;
  size_t nblk = (size_t)n_out * (k_in / 32);
  Q8View v;
  v.qs = (const int8_t*)p;
  v.d = (const uint16_t*)(p + up256(nblk * 32));
  v.nb = k_in / 32;
  v.n_out = n_out;
  return v;
}

// ------------------------------------------------------- activation images
// Rows of activations prepared for the fp16 matrix cores.  Every row is
// scaled by its own power of two 2^e (its largest magnitude lands in
// [2^10, 2^11), far from fp16 overflow even after 16-element sums) and split
// into an fp16 high part and an fp16 remainder (~22 significant bits
// together; a bf16 row is exact in the high part alone).  rscale holds 2^-e
// per row; consumers multiply their finished sums by it, so the scaling is
// exact end to end.
//  layout PERM (two-bit kernels): element order matches the register order in
//    which the two-bit kernel unpacks codes, with the 4^-j factor of each
//    position folded in; plus per-16-element sums (for the min term), stored
//    per group of 4 sub-blocks as their 4 high parts then their 4 remainders
//    (the order the kernel reads them in).
//  layout PLAIN (eight-bit kernel): natural order.
struct XImg {
  _Float16* hi;      // [rows, K]
  _Float16* lo;      // [rows, K]
  _Float16* sx;      // [rows, K/8]  (PERM only)
  float* rscale;     // [rows]  2^-e
  int K;
};

enum { XL_PERM = 0, XL_PLAIN = 1 };

__host__ __device__ inline size_t ximg_bytes(size_t rows, size_t K, int layout) {
  size_t b = 2 * up256(rows * K * 2) + up256(rows * 4);
  if (layout == XL_PERM) b += up256(rows * (K / 8) * 2);
  return b;
}

inline XImg ximg_carve(void* base, size_t rows, int K, int layout) {
  uint8_t* p = (uint8_t*)base;
  XImg x;
  x.K = K;
  x.hi = (_Float16*)p;
  p += up256(rows * K * 2);
  x.lo = (_Float16*)p;
  p += up256(rows * K * 2);
  if (layout == XL_PERM) {
    x.sx = (_Float16*)p;
    p += up256(rows * (K / 8) * 2);
  } else {
    x.sx = nullptr;
  }
  x.rscale = (float*)p;
  return x;
}

// ------------------------------------------------------ activation digits
// Rows prepared for the int8 matrix cores: each row r is scaled by its own
// power of two 2^s_r (its largest magnitude lands in [2^29, 2^30)), rounded to
// integers a and written as four signed bytes a = 2^24 p0 + 2^16 p1 + 2^8 p2 +
// p3 (balanced digits: p1..p3 in -128..127, |p0| <= 64).  Plane i holds digit
// p_i of every element, in the byte order the two-bit contraction consumes:
// byte kb*256 + 64 t + 16 g + 4 j + b <-> element kb*256 + (4g + t)*16 + 4b + j
// (block kb, sub-block 4g + t, the 16 bytes one lane group reads at step t).
// sx holds each digit plane's sums over the 16 elements of a sub-block (exact
// integers, |sum| <= 2048, exact in fp16) for the min term.  rsc = 2^-s_r, or
// NaN for a row with a non-finite value (whose digits are all zero).
struct XDig {
  int8_t* dig;      // [rows][4][K]
  _Float16* sx;     // [rows][4][K/16]
  float* rsc;       // [rows]
  int K;
};

__host__ __device__ inline size_t xdig_bytes(size_t rows, size_t K) {
  return up256(rows * 4 * K) + up256(rows * 4 * (K / 16) * 2) + up256(rows * 4);
}

inline XDig xdig_carve(void* base, size_t rows, int K) {
  uint8_t* p = (uint8_t*)base;
  XDig x;
  x.K = K;
  x.dig = (int8_t*)p;
  p += up256(rows * 4 * K);
  x.sx = (_Float16*)p;
  p += up256(rows * 4 * (K / 16) * 2);
  x.rsc = (float*)p;
  return x;
}

// ----------------------------------------------------------- MoE workspace
// Device-side routing/grouping results written by the prep kernel.
struct MoeMeta {
  int n_units;    // touched routed experts + shared
  int n_assign;   // (row, slot) assignments incl. shared rows
  int n_work_gu;  // descriptors of the gate/up kernel
  int n_work_dn;  // descriptors of the down kernel
};

// One descriptor of the expert kernels: a column group of one unit (an
// expert, -1 = shared): its first assignment a0, its ncols assignments and
// the activation row of each.  type (gate/up): MOE_ALLK -- the rows' digits
// over all of K stay resident and the block's waves split K; MOE_QUARTER --
// the block's waves take four tiles of one quarter of K.  Either way the
// quarter sums go to the workspace and SwiGLU happens when the down
// projection's input is staged (k_hdig).  Down descriptors carry their unit's
// gate/up type.  One 48-byte load per descriptor.
constexpr int MOE_WORK_COLS = 8;
constexpr int MOE_MAX_GRID = 1024;   // persistent blocks of an expert kernel, at most
// Relative cost of an expert-kernel item whose descriptor has at most four
// rows (one column tile) and more (two column tiles, the weight tile shared),
// as measured per kernel: the block ranges are cut to equal cost with these
// weights.
constexpr int MOE_COST_1 = 10;
constexpr int MOE_COST_2_GU = 16, MOE_COST_2_DN = 19;
// Cost of a block's change of descriptor inside its range (a barrier, at
// which the waves that run ahead wait for the others, the new rows' copy,
// and the load ring drained), on the same scale, charged at the start of
// every descriptor: measured for gate/up (about 0.8 of an item); for down
// (about 0.35) charging it made no difference.
constexpr int MOE_SWITCH_GU = 8, MOE_SWITCH_DN = 0;
enum { MOE_ALLK = 0, MOE_QUARTER = 1 };
struct MoeWork {
  int expert, a0, ncols, type;
  int rows[MOE_WORK_COLS];
};

struct MoeWs {
  MoeMeta* meta;
  int* unit_expert;   // [max_units]  expert id, -1 = shared
  int* unit_off;      // [max_units]  first assignment of the unit
  int* unit_cnt;      // [max_units]
  int* arow;          // [max_assign] activation row of assignment a
  int* amap;          // [R, top_k+1]  assignment of (row, slot); slot top_k = shared
  int* topk_idx;      // [R, top_k]
  float* topk_w;      // [R, top_k]
  float* gpart;       // [2][4][max_assign, inter]  gate / up quarter sums
  float* part;        // [max_assign, hidden] per-assignment down outputs
  MoeWork* work_gu;   // [max_work]
  MoeWork* work_dn;   // [max_work]
  int* blk_gu;        // [MOE_MAX_GRID + 1] first item of each persistent gate/up block
  int* blk_dn;        // [MOE_MAX_GRID + 1] the same for the down kernel
  XDig hd;            // the down projection's input rows as digits  [max_assign, inter]
  XDig xd;            // x as digits  [R, hidden]
  XImg x_img;         // x staged for the one-matrix (PLAIN) path  [R, hidden]
  // eight-bit shared expert: x and h staged for the head kernels; the gate and
  // up products as sums of sp_gu slices over K ([2][sp_gu][R, inter]), the
  // down product as sp_dn slices ([sp_dn][R, hidden])
  XImg sx_img, sh_img;
  float *sgu, *sdn;
  int sp_gu, sp_dn;
  int max_units, max_assign, max_work;
};

// Whether the layer's shared expert runs on the eight-bit path.
inline bool shared_q8(const sv_moe_desc* d) {
  return d->ffn == SV_FFN_SWIGLU && d->s_gate != nullptr && d->s_format == SV_Q8;
}

size_t moe_ws_layout(const sv_moe_desc* d, int R, void* base, MoeWs* out);

// Compute units of the current device (cached per device; 256 if the query
// fails).  Persistent kernels size their grids with it; any value is correct,
// only the speed depends on it.
int cu_count();

// ------------------------------------------------------------- launchers
// All return hipSuccess or the launch error.
hipError_t launch_stage(const void* src, int dtype, int rows, int K, int layout,
                        const int* n_rows_dev, XImg img, hipStream_t s);
hipError_t launch_moe_prep(const sv_moe_desc* d, int R, const float* router_logits,
                           const void* x, int x_dtype, int32_t* topk_idx_out,
                           float* topk_w_out, MoeWs ws, hipStream_t s);
hipError_t launch_q2_plain(const sv_moe_desc* d, int R, bool use_lo, MoeWs ws, float* y,
                           hipStream_t s);
// Persistent blocks of the expert kernels (the device's compute units, at
// most MOE_MAX_GRID).
int moe_grid();
hipError_t launch_moe_gateup(const sv_moe_desc* d, int R, MoeWs ws, hipStream_t s);
hipError_t launch_hdig(const sv_moe_desc* d, int R, MoeWs ws, hipStream_t s);
hipError_t launch_moe_down(const sv_moe_desc* d, int R, MoeWs ws, hipStream_t s);
hipError_t launch_moe_combine(const sv_moe_desc* d, int R, MoeWs ws, float* y, hipStream_t s);
// The eight-bit shared expert: its K-slice counts (ws->sp_gu, sp_dn), then its
// products into ws.sgu / ws.sdn (k_moe_combine adds the down slices).
void plan_shared_q8(const sv_moe_desc* d, int R, int x_dtype, MoeWs* ws);
hipError_t launch_shared_q8(const sv_moe_desc* d, int R, const void* x, int x_dtype, MoeWs ws,
                            hipStream_t s);
// K slices of the head kernel's split form for [vocab x hidden] on R rows and
// nmat matrices (0: the split form does not take this shape), and its launch
// (w2 may be null): partial products [nmat][slices][R, vocab] into part.
int q8_split_parts(int vocab, int hidden, int R, bool use_lo, int nmat);
hipError_t launch_q8_split(const void* w1, const void* w2, int vocab, int hidden, int R, bool use_lo, XImg img,
                           float* part, hipStream_t s);
// Whether the streamed int8 expert kernels take this layer (LDS limits).
bool moe_shape_ok(const sv_moe_desc* d);
hipError_t launch_q2_tile(const void* src, void* dst, int n_out, int k_in, int parts, int count, hipStream_t s);
hipError_t launch_q8_lmhead(const void* w, int vocab, int hidden, int R, bool use_lo,
                            XImg img, float* logits, hipStream_t s);
hipError_t launch_accept(int S, int K, int V, const float* target, int tkind, float Tp,
                         const float* draft, int dkind, float Tq, const int32_t* drafts,
                         const float* u, int32_t* out_tokens, int32_t* out_n, void* ws,
                         hipStream_t s);
size_t accept_ws_bytes(int S, int K, int V);
hipError_t launch_accept_tsm(int S, int K, int V, const float* target, int tkind, float Tp,
                             const int32_t* drafts, const float* u, int32_t* out_tokens, int32_t* out_n,
                             void* ws, hipStream_t s);
size_t accept_tsm_ws_bytes(int S, int K, int V);
hipError_t launch_read_probe(const void* src, size_t bytes, int mode, uint32_t* sink, hipStream_t s);
size_t read_probe_sink_words();
hipError_t launch_q2_dequant(const void* w, int n_out, int k_in, float* out, hipStream_t s);
hipError_t launch_q8_dequant(const void* w, int n_out, int k_in, float* out, hipStream_t s);

}  // namespace sv

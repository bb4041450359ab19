// Read-bandwidth probe: streams a buffer once with one of a few access
// patterns, so that the part's attainable read rate -- the denominator the
// roofline fractions are read against ("ds4-on-spark" README, "Roofline: why
// speculation and batching are the levers": a measured bandwidth, not the
// data-sheet figure) -- is measured with the same instructions the weight
// kernels use.
//
// The buffer is viewed as groups of 16 rows x 1792 bytes (the code plane of a
// 16-row tile of a 7168-wide two-bit matrix: 28 blocks of 64 bytes per row).
// Every wave owns a contiguous range of groups and reads each group with 28
// wave instructions of 1 KB (64 lanes x 16 bytes), keeping PROBE_DEPTH of them
// in flight:
//   mode 0  plain loads into registers, full 128-byte lines (8 rows x 128 B
//           per instruction: the two-block step)
//   mode 1  global-to-LDS loads, non-temporal, full lines (as mode 0)
//   mode 2  global-to-LDS loads, full lines, default cache policy
//   mode 3  global-to-LDS loads, 64-byte pieces (16 rows x 64 B per
//           instruction: the one-block step; the other half of every line is
//           read by the next instruction)
//   mode 4  as mode 3, non-temporal
//   mode 5  global-to-LDS 4-byte loads, non-temporal, 256 contiguous bytes per
//           instruction (the pattern of the small scale planes)
// One dword per wave goes to `sink` so that no load is dead.
#include "sv_internal.h"

namespace sv {

constexpr int PROBE_ROW = 1792, PROBE_GROUP = 16 * PROBE_ROW, PROBE_DEPTH = 8;

__device__ __forceinline__ void probe_dma4(const void* src, uint32_t la) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off nt"
               :: "v"(src), "s"(__builtin_amdgcn_readfirstlane(la)) : "memory", "m0");
}

__device__ __forceinline__ void probe_dma(const void* src, uint32_t la, bool nt) {
  if (nt)
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt"
                 :: "v"(src), "s"(__builtin_amdgcn_readfirstlane(la)) : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(src), "s"(__builtin_amdgcn_readfirstlane(la)) : "memory", "m0");
}

// Byte offset, inside a group, of lane `lane`'s 16 bytes of instruction j.
__device__ __forceinline__ uint32_t probe_off(int mode, int j, int lane) {
  if (mode == 5) return 256 * j + 4 * lane;   // (the first 7 KB of the group, 4 B per lane)
  if (mode == 3 || mode == 4) {   // 16 rows x 64 B at column 64 j
    const int row = lane >> 2, q = lane & 3;
    return row * PROBE_ROW + 64 * j + 16 * q;
  }
  // 8 rows x 128 B: rows 8 (j & 1) .. +7 at column 128 (j >> 1)
  const int row = 8 * (j & 1) + (lane >> 3), q = lane & 7;
  return row * PROBE_ROW + 128 * (j >> 1) + 16 * q;
}

template <int MODE>
__global__ __launch_bounds__(256) void k_read_probe(const uint8_t* src, long ngroups, uint32_t* sink) {
  __shared__ __align__(16) uint8_t ring[4][PROBE_DEPTH][1024];
  const int lane = threadIdx.x & 63, wv = wave_id();
  const long nw = (long)gridDim.x * 4, w = (long)blockIdx.x * 4 + wv;
  const long g0 = ngroups * w / nw, g1 = ngroups * (w + 1) / nw;
  const uint32_t lbase = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)&ring[wv][0][0];
  uint32_t acc = 0;
  int slot = 0;
  for (long g = g0; g < g1; ++g) {
    const uint8_t* gp = src + g * PROBE_GROUP;
#pragma unroll
    for (int j = 0; j < 28; ++j) {
      const uint8_t* p = gp + probe_off(MODE, j, lane);
      if (MODE == 0) {
        const uint4 v = *(const uint4*)p;
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
      } else if (MODE == 5) {
        probe_dma4(p, lbase + slot * 1024);
        slot = (slot + 1) & (PROBE_DEPTH - 1);
        wait_vmcnt_le(PROBE_DEPTH - 1);
      } else {
        probe_dma(p, lbase + slot * 1024, MODE == 1 || MODE == 4);
        slot = (slot + 1) & (PROBE_DEPTH - 1);
        wait_vmcnt_le(PROBE_DEPTH - 1);
      }
    }
  }
  wait_vmcnt_le(0);
  if (MODE != 0) acc = ((const uint32_t*)&ring[wv][0][0])[lane];
  acc = wave_allreduce(acc, [](uint32_t a, uint32_t b) { return a ^ b; });
  if (lane == 0) sink[w] = acc;
}

hipError_t launch_read_probe(const void* src, size_t bytes, int mode, uint32_t* sink, hipStream_t s) {
  const long ngroups = (long)(bytes / PROBE_GROUP);
  const dim3 grid(2 * cu_count()), block(256);
  const uint8_t* p = (const uint8_t*)src;
  switch (mode) {
    case 0: hipLaunchKernelGGL(k_read_probe<0>, grid, block, 0, s, p, ngroups, sink); break;
    case 1: hipLaunchKernelGGL(k_read_probe<1>, grid, block, 0, s, p, ngroups, sink); break;
    case 2: hipLaunchKernelGGL(k_read_probe<2>, grid, block, 0, s, p, ngroups, sink); break;
    case 3: hipLaunchKernelGGL(k_read_probe<3>, grid, block, 0, s, p, ngroups, sink); break;
    case 4: hipLaunchKernelGGL(k_read_probe<4>, grid, block, 0, s, p, ngroups, sink); break;
    default: hipLaunchKernelGGL(k_read_probe<5>, grid, block, 0, s, p, ngroups, sink); break;
  }
  return hipGetLastError();
}

size_t read_probe_sink_words() { return (size_t)2 * cu_count() * 4; }

}  // namespace sv

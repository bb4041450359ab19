// Activation rows as signed byte digits for the int8 matrix cores (layout in
// sv_internal.h, struct XDig).  A row's values are scaled by one power of two
// 2^s (its largest magnitude lands in [2^29, 2^30)) and rounded to integers a;
// every a is written as a = 2^24 p0 + 2^16 p1 + 2^8 p2 + p3 with p1, p2, p3 in
// -128..127 and |p0| <= 64.  The only rounding is a's: |x - a 2^-s| <=
// 2^-(s+1), i.e. at most 2^-30 of the row's largest magnitude -- bf16 values
// within 2^-22 of the row's maximum are exact, fp32 values lose at most the
// bits below 2^-30 of it.
#pragma once

#include "sv_internal.h"

namespace sv {

// Signed byte with the low 8 bits of x (sign-extended).
__device__ __forceinline__ int sbyte(int x) { return (x << 24) >> 24; }

constexpr int NDIG = 4;   // digit planes per row

// Scale exponent of a row whose largest magnitude is mx: mx 2^s in
// [2^29, 2^30); 0 for an all-zero row.
__device__ __forceinline__ int digit_exponent(float mx) {
  if (!(mx > 0.f)) return 0;
  int E;
  frexpf(mx, &E);   // mx in [2^(E-1), 2^E)
  return min(max(30 - E, -120), 120);
}

// The 16 values of one sub-block as digits: the sub-block's 16 bytes of each
// of the four planes (byte 4j + b <-> value 4b + j) and the four digit sums.
// bad: the row holds a non-finite value; its digits are all zero.
__device__ __forceinline__ void subblock_digits(const float (&v)[16], int s, bool bad, uint4 (&pl)[NDIG],
                                                int (&sums)[NDIG]) {
  uint32_t w[NDIG][4];
#pragma unroll
  for (int i = 0; i < NDIG; ++i) {
    sums[i] = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[i][j] = 0u;
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int a = bad ? 0 : (int)rintf(ldexpf(v[e], s));
    const int p3 = sbyte(a), a1 = (a - p3) >> 8;
    const int p2 = sbyte(a1), a2 = (a1 - p2) >> 8;
    const int p1 = sbyte(a2), p0 = (a2 - p1) >> 8;
    const int dg[NDIG] = {p0, p1, p2, p3};
    const int j = e & 3, b = e >> 2;
#pragma unroll
    for (int i = 0; i < NDIG; ++i) {
      w[i][j] |= ((uint32_t)dg[i] & 0xFFu) << (8 * b);
      sums[i] += dg[i];
    }
  }
#pragma unroll
  for (int i = 0; i < NDIG; ++i) pl[i] = make_uint4(w[i][0], w[i][1], w[i][2], w[i][3]);
}

// Byte offset of sub-block sb (of the whole row) inside a digit plane.
__host__ __device__ __forceinline__ size_t subblock_offset(int sb) {
  const int kb = sb >> 4, sl = sb & 15;
  return (size_t)kb * 256 + 64 * (sl & 3) + 16 * (sl >> 2);
}

}  // namespace sv

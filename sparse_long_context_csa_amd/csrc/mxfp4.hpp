// MXFP4 storage of indexer keys: E2M1 elements, one E8M0 scale per 32 channels.
//
// "DeepSeek V4-Flash: The Cost of Deciding What to Read", section "What the cache costs,
// checked four ways" (the indexer cache is FP4: 64 bytes per 128-channel key) and section "FP4,
// down to the index scores" (1 x 32 MXFP4 sub-blocks). Format as in the OCP microscaling
// definition: element = sign, 2 exponent bits (bias 1), 1 mantissa bit (magnitudes 0, 0.5, 1,
// 1.5, 2, 3, 4, 6); block scale 2^(s - 127) stored as the byte s. Quantisation: s = floor(log2
// max|x|) - 2 clamped to [-127, 127] (-127 for a zero block); x / 2^s rounds to the nearest
// magnitude, ties to the even code, past 6 to 6; a zero magnitude is code 0. Element 2i sits in
// the low nibble of byte i.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace csa {

// shared exponent of a block with largest magnitude amax (exact: frexp is exact)
__device__ __forceinline__ int mx_shared_exp(float amax) {
  if (!(amax > 0.f)) return -127;
  int e;
  (void)frexpf(amax, &e);           // amax = f 2^e, f in [0.5, 1): floor(log2 amax) = e - 1
  const int s = e - 1 - 2;
  return s < -127 ? -127 : (s > 127 ? 127 : s);
}

// E2M1 code of v (already divided by the block scale): nearest magnitude, ties to the even
// code. The code is the number of midpoints between magnitudes (exact in binary) that |v| has
// reached; at a midpoint the count stops at the even code of its two neighbours, so those below
// an even code (0.75, 1.75, 3.5) count once reached and the others once passed. Summed
// comparisons, no branches.
__device__ __forceinline__ uint32_t e2m1_code(float v) {
  const float a = fabsf(v);
  const uint32_t c = uint32_t(a > 0.25f) + uint32_t(a >= 0.75f) + uint32_t(a > 1.25f) +
                     uint32_t(a >= 1.75f) + uint32_t(a > 2.5f) + uint32_t(a >= 3.5f) +
                     uint32_t(a > 5.f);
  return c | (uint32_t(v < 0.f && c != 0u) << 3);
}

// value of an E2M1 code times 2^(s - 127) (exact in fp32 and in bf16)
__device__ __forceinline__ float e2m1_value(uint32_t code, uint32_t s) {
  const uint32_t m = code & 7u;
  const float mag = m < 2u ? 0.5f * float(m) : float((2u + (m & 1u)) << ((m >> 1) - 1u)) * 0.5f;
  const float sc = __uint_as_float(s == 0u ? 0x00400000u : (s << 23));   // 2^(s - 127)
  return (code & 8u) ? -mag * sc : mag * sc;
}

}  // namespace csa

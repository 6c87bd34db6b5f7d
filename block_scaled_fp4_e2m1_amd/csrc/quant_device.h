// Device-side block quantisation helpers (E4M3 / E8M0 / E2M1 encoders) shared
// by the quantiser kernel and the fused MoE activation epilogue, so that both
// produce the same bytes.  Every step is one correctly rounded binary32
// operation; the sources that include this header are compiled with
// -ffp-contract=off and correctly rounded division.
#pragma once

#include "device_common.h"

#pragma clang fp contract(off)

namespace bsfp4 {

// Nearest-even E4M3 code of s >= 0, saturating to 0x7E (448) instead of NaN.
__device__ __forceinline__ uint32_t e4m3_rne_satfinite(float s) {
  if (!(s < 448.0f)) return 0x7Eu;
  if (s < 0.015625f) {
    // Subnormal range (below 2^-6): the grid is k * 2^-9, k = 0..8, and
    // k = 8 is the bit pattern of 2^-6 itself.  s * 512 is exact.
    return (uint32_t)__builtin_rintf(s * 512.0f);
  }
  const uint32_t u = __float_as_uint(s);
  const uint32_t e = (u >> 23) - 120u;  // E4M3 biased exponent (bias 7), 1..15
  const uint32_t keep = (u >> 20) & 7u;  // top three mantissa bits
  const uint32_t rest = u & 0xFFFFFu;    // the 20 bits rounded away
  uint32_t code = (e << 3) | keep;
  code += (rest > 0x80000u) || (rest == 0x80000u && (keep & 1u));  // may carry into e
  return code;
}

__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  const uint32_t e = c >> 3, m = c & 7u;
  if (e == 0) return (float)m * 0.001953125f;          // m * 2^-9
  return __uint_as_float(((e + 120u) << 23) | (m << 20));  // (1 + m/8) * 2^(e-7)
}

// Smallest power of two >= s (s >= 0) as an E8M0 code in [0, 254].
__device__ __forceinline__ uint32_t e8m0_ceil(float s) {
  const uint32_t u = __float_as_uint(s);
  const uint32_t ef = u >> 23, m = u & 0x7FFFFFu;
  if (ef == 0) return m > 0x400000u ? 1u : 0u;  // binary32 subnormal: 2^-127 = m of 2^22
  const uint32_t c = ef + (m != 0u);
  return c > 254u ? 254u : c;
}

// 2^(127 - c) for an E8M0 code c in [0, 254] (2^-127 is a binary32 subnormal).
__device__ __forceinline__ float e8m0_inverse(uint32_t c) {
  return c == 254u ? __uint_as_float(0x00400000u) : __uint_as_float((254u - c) << 23);
}

// Nearest-even E2M1 code of y, saturating at 6, keeping the sign bit.  The
// magnitude code counts the midpoints |y| has passed; at a midpoint the
// neighbour with mantissa bit 0 wins, hence the alternating > / >=.
__device__ __forceinline__ uint32_t e2m1_rne(float y) {
  const float a = fabsf(y);
  const uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                     (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                     (uint32_t)(a > 5.0f);
  return c | ((__float_as_uint(y) >> 28) & 8u);
}

// Quantise 32 binary32 values (one MXFP4 block) to 16 code bytes (4 words) and
// return the E8M0 scale code.
__device__ __forceinline__ uint32_t mxfp4_block32(const float (&v)[32], uint32_t (&packed)[4]) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; i++) amax = fmaxf(amax, fabsf(v[i]));
  const uint32_t scode = e8m0_ceil(amax / 6.0f);
  const float inv = e8m0_inverse(scode);
#pragma unroll
  for (int j = 0; j < 4; j++) {
    uint32_t word = 0;
#pragma unroll
    for (int t = 0; t < 8; t++) word |= e2m1_rne(v[8 * j + t] * inv) << (4 * t);
    packed[j] = word;
  }
  return scode;
}

}  // namespace bsfp4

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

// E2M1 codes of two values into byte `sel` of `word` (first value in the low
// nibble) with gfx950's v_cvt_scalef32_pk_fp4_*: nearest-even, ties to the
// even code, saturating at 6, the sign bit kept (so -0 and negatives that
// round to zero give code 8).  These are the encoder's rules: E2M1 magnitudes
// {0, 0.5, 1, 1.5, 2, 3, 4, 6} with midpoints 0.25, 0.75, 1.25, 1.75, 2.5,
// 3.5, 5 rounding to the code with mantissa bit 0.  The three helpers below
// are exported unchanged through bsfp4_e2m1_convert, and the GPU test
// tests/test_gpu_e2m1_converters.py holds them bit for bit to the oracle's
// encoder: every non-NaN bf16 pattern at several E8M0 scales, every E2M1
// midpoint and grid point +-1..3 ulp, subnormals, +-0, +-inf and dense random
// binary32 sweeps (NaN inputs are outside the contract).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// codes of (a, b), scale 1
__device__ __forceinline__ uint32_t e2m1x2_f32(uint32_t word, float a, float b, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, a, b, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, a, b, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, a, b, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, a, b, 1.0f, 3);
  }
}

// codes of the two bf16 values in `pair` (low half first) divided by
// 2^(scode - 127), an E8M0 scale (2^-127 is a binary32 subnormal; the
// instruction takes it as it is)
__device__ __forceinline__ uint32_t e2m1x2_bf16_pow2(uint32_t word, uint32_t pair, uint32_t scode, int sel) {
  const float scale = __uint_as_float(scode == 0 ? 0x00400000u : scode << 23);
  const bf16x2_t v = __builtin_bit_cast(bf16x2_t, pair);
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(word, v, scale, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(word, v, scale, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(word, v, scale, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(word, v, scale, 3);
  }
}

// codes of the binary32 values (a, b) divided by 2^(scode - 127), an E8M0
// scale (the MXFP4 re-quantisation of the fused SiLU-mul epilogue)
__device__ __forceinline__ uint32_t e2m1x2_f32_pow2(uint32_t word, float a, float b, uint32_t scode, int sel) {
  const float scale = __uint_as_float(scode == 0 ? 0x00400000u : scode << 23);
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, a, b, scale, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, a, b, scale, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, a, b, scale, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, a, b, scale, 3);
  }
}

}  // namespace bsfp4

// Device-side helpers shared by the gfx950 kernels of libbsfp4.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsfp4 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b) {
  return __uint_as_float(b << 16);
}

// Round-to-nearest-even of a finite binary32 to bf16 bits (NaN not handled:
// the kernels never produce one from finite inputs).
__device__ __forceinline__ uint32_t float_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two binary32 values -> packed bf16 pair (first in the low half), RNE.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return float_to_bf16_rne(lo) | (float_to_bf16_rne(hi) << 16);
}

// E4M3 scale code (magnitude bits) -> its value in binary32, exact and without
// a branch: the 7 magnitude bits placed at fp16 bit 7 are the E4M3 value times
// 2^-8 for normal and subnormal codes alike.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)((c & 0x7Fu) << 7));
  return (float)h * 256.0f;
}

// Eight E2M1 values (one 32-bit word, first value in the low nibble) times the
// binary32 block scale `s` -> eight bf16 values.  The products have at most 6
// significant bits, so they are exact in binary32 and in bf16.
__device__ __forceinline__ v8bf dq8_bf16(uint32_t word, float s) {
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    v2f f;
    switch (j) {
      case 0: f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 0); break;
      case 1: f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 1); break;
      case 2: f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 2); break;
      default: f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 3); break;
    }
    // exact products, so the nearest-even conversion is exact
    o[j] = __builtin_bit_cast(uint32_t, v2bf{(__bf16)(f.x * s), (__bf16)(f.y * s)});
  }
  return __builtin_bit_cast(v8bf, make_uint4(o[0], o[1], o[2], o[3]));
}

// E4M3 byte -> fp16 (exact): the 7 magnitude bits at fp16 bit 7 give the value
// times 2^-8 for normal and subnormal codes; multiplying by 256 restores it.
__device__ __forceinline__ _Float16 e4m3_to_f16(uint32_t c) {
  const uint16_t bits = (uint16_t)((c & 0x7Fu) << 7);
  return __builtin_bit_cast(_Float16, bits) * (_Float16)256.0f;
}

// Eight E2M1 values (one 32-bit word, first value in the low nibble) times the
// fp16 block scale `s` -> eight fp16 values (exact: at most 6 significant bits,
// magnitudes in [2^-10, 2688]).
__device__ __forceinline__ v8h dq8_f16(uint32_t word, _Float16 s) {
  const v2h ss = {s, s};
  const v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 0) * ss;
  const v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 1) * ss;
  const v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 2) * ss;
  const v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 3) * ss;
  const v4h lo = __builtin_shufflevector(p0, p1, 0, 1, 2, 3);
  const v4h hi = __builtin_shufflevector(p2, p3, 0, 1, 2, 3);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

}  // namespace bsfp4

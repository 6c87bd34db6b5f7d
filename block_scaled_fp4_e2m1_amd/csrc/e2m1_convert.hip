// Exported E2M1 conversion: the device routines with which the quantiser and
// the fused SiLU-mul + MXFP4 epilogue turn values into E2M1 codes, run on
// caller-given values.  The pages name the per-block quant routine
// (`cvt_warp_fp16_to_fp4`, `cvt_fp16_to_fp4_sm103` on the vLLM `sm103` branch
// comparison page) but do not print its body, so the rounding rule is this
// library's reading (nearest, ties to the even code, saturation at 6, sign
// kept); this entry point lets a test hold the hardware converters to a
// reference encoder over whole input classes.
#include "device_common.h"
#include "launchers.h"
#include "quant_device.h"

namespace bsfp4 {
namespace {

// One output dword = 4 pairs, pair j in byte j (the same byte-select operand
// the kernels use).  MODE 0: binary32 pairs, scale 1.  MODE 1: bf16 pairs
// divided by 2^(scale code - 127).  MODE 2: binary32 pairs divided by
// 2^(scale code - 127).
template <int MODE>
__global__ void __launch_bounds__(256)
    e2m1_convert(const uint32_t* __restrict__ in, const uint8_t* __restrict__ scodes, uint32_t* __restrict__ out,
                 int64_t words) {
  for (int64_t w = (int64_t)blockIdx.x * 256 + threadIdx.x; w < words; w += (int64_t)gridDim.x * 256) {
    uint32_t word = 0;
    if constexpr (MODE == 1) {
      const uint4 v = reinterpret_cast<const uint4*>(in)[w];
      const uint32_t s = reinterpret_cast<const uint32_t*>(scodes)[w];
      word = e2m1x2_bf16_pow2(word, v.x, s & 0xFFu, 0);
      word = e2m1x2_bf16_pow2(word, v.y, (s >> 8) & 0xFFu, 1);
      word = e2m1x2_bf16_pow2(word, v.z, (s >> 16) & 0xFFu, 2);
      word = e2m1x2_bf16_pow2(word, v.w, s >> 24, 3);
    } else {
      const uint4 v0 = reinterpret_cast<const uint4*>(in)[2 * w];
      const uint4 v1 = reinterpret_cast<const uint4*>(in)[2 * w + 1];
      const float f[8] = {__uint_as_float(v0.x), __uint_as_float(v0.y), __uint_as_float(v0.z),
                          __uint_as_float(v0.w), __uint_as_float(v1.x), __uint_as_float(v1.y),
                          __uint_as_float(v1.z), __uint_as_float(v1.w)};
      if constexpr (MODE == 0) {
        word = e2m1x2_f32(word, f[0], f[1], 0);
        word = e2m1x2_f32(word, f[2], f[3], 1);
        word = e2m1x2_f32(word, f[4], f[5], 2);
        word = e2m1x2_f32(word, f[6], f[7], 3);
      } else {
        const uint32_t s = reinterpret_cast<const uint32_t*>(scodes)[w];
        word = e2m1x2_f32_pow2(word, f[0], f[1], s & 0xFFu, 0);
        word = e2m1x2_f32_pow2(word, f[2], f[3], (s >> 8) & 0xFFu, 1);
        word = e2m1x2_f32_pow2(word, f[4], f[5], (s >> 16) & 0xFFu, 2);
        word = e2m1x2_f32_pow2(word, f[6], f[7], s >> 24, 3);
      }
    }
    out[w] = word;
  }
}

}  // namespace

hipError_t launch_e2m1_convert(int mode, const void* in, const uint8_t* scale_codes, int64_t pairs,
                               uint8_t* codes, hipStream_t stream) {
  const int64_t words = pairs / 4;
  if (words == 0) return hipSuccess;
  const int64_t g = (words + 255) / 256;
  const unsigned grid = (unsigned)(g > 4096 ? 4096 : g);
  const uint32_t* src = static_cast<const uint32_t*>(in);
  uint32_t* dst = reinterpret_cast<uint32_t*>(codes);
  switch (mode) {
    case 0: e2m1_convert<0><<<grid, 256, 0, stream>>>(src, scale_codes, dst, words); break;
    case 1: e2m1_convert<1><<<grid, 256, 0, stream>>>(src, scale_codes, dst, words); break;
    default: e2m1_convert<2><<<grid, 256, 0, stream>>>(src, scale_codes, dst, words); break;
  }
  return hipGetLastError();
}

}  // namespace bsfp4

// On-box peak probes: the rates that the roofline fractions of the hot-path
// kernels are also reported against, measured on the device that runs them
// (the published MI355X figures are the primary denominators).
//
//   mfma_probe<KIND>  every wave keeps 8 independent 32x32 accumulators and
//                     issues MFMAs back to back from registers (no memory
//                     traffic): KIND 0 fp16 32x32x16, 1 bf16 32x32x16,
//                     2 fp8 (E4M3) 32x32x64, 3 fp4 (E2M1, E8M0 scale 1.0)
//                     32x32x64 scaled MFMA; 4 and 5 are fp16 and bf16 with
//                     operands of at most 3 significant bits (as the exactly
//                     dequantised E2M1 x E4M3 values have few), since the
//                     sustained MFMA rate of a power-limited part depends on
//                     how many operand bits toggle.  6 and 7 feed operands
//                     that change from one MFMA to the next, as in a GEMM
//                     (four A and four B registers, rotated): 6 fp4 with
//                     random codes, 7 fp16 with random E2M1 x E4M3 products
//                     (the values the exact NVFP4 path multiplies).  Four
//                     256-thread workgroups per compute unit.
//   read_probe        streams a buffer once with 128-bit loads (four in
//                     flight per lane), keeping a running XOR; nothing is
//                     stored unless the flag (never set by the library) asks.
#include "device_common.h"
#include "launchers.h"

namespace bsfp4 {
namespace {

// 32-bit linear congruential step (Numerical Recipes constants) with an
// xor-shift of the output: operand bits for the changing-operand kinds
__device__ __forceinline__ uint32_t lcg_next(uint32_t& s) {
  s = s * 1664525u + 1013904223u;
  return s ^ (s >> 13);
}

template <int KIND>
__global__ void __launch_bounds__(256) mfma_probe(int iters, int flag, float* sink) {
  const int lane = threadIdx.x & 63;
  v16f acc[8];
#pragma unroll
  for (int j = 0; j < 8; j++) acc[j] = v16f{};
  if constexpr (KIND >= 6) {
    // four A and four B operands per lane; MFMA j of step u multiplies A j%4
    // by B (j/2 + u)%4, so consecutive MFMAs never repeat an operand pair
    uint32_t st = 0x9e3779b9u * (threadIdx.x + 1) + blockIdx.x * 7919u;
    if constexpr (KIND == 6) {
      v8i a[4], b[4];
#pragma unroll
      for (int j = 0; j < 4; j++)
#pragma unroll
        for (int i = 0; i < 8; i++) {
          a[j][i] = i < 4 ? (int)lcg_next(st) : 0;
          b[j][i] = i < 4 ? (int)lcg_next(st) : 0;
        }
      for (int it = 0; it < iters; it += 4) {
#pragma unroll
        for (int u = 0; u < 4; u++)
#pragma unroll
          for (int j = 0; j < 8; j++)
            acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[j & 3], b[((j >> 1) + u) & 3], acc[j], 4, 4,
                                                                     0, 127, 0, 127);
      }
    } else {
      const float e2[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
      v8h a[4], b[4];
#pragma unroll
      for (int j = 0; j < 4; j++)
#pragma unroll
        for (int i = 0; i < 8; i++) {
          // E2M1 value x E4M3 mantissa (1 + m/8) x 2^(0..3) x sign / 8
          uint32_t r = lcg_next(st);
          a[j][i] = (_Float16)(e2[r & 7] * (1.0f + 0.125f * ((r >> 3) & 7)) * (float)(1 << ((r >> 6) & 3)) *
                               (((r >> 9) & 1) ? -0.125f : 0.125f));
          r = lcg_next(st);
          b[j][i] = (_Float16)(e2[r & 7] * (1.0f + 0.125f * ((r >> 3) & 7)) * (float)(1 << ((r >> 6) & 3)) *
                               (((r >> 9) & 1) ? -0.125f : 0.125f));
        }
      for (int it = 0; it < iters; it += 4) {
#pragma unroll
        for (int u = 0; u < 4; u++)
#pragma unroll
          for (int j = 0; j < 8; j++)
            acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[j & 3], b[((j >> 1) + u) & 3], acc[j], 0, 0, 0);
      }
    }
  } else if constexpr (KIND <= 1 || KIND >= 4) {
    v8h a, b;
    v8bf ab, bb;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      float x, y;
      if constexpr (KIND >= 4) {
        // (1 + m/4) * 2^e, m in 0..3, |e| <= 3: at most 3 significant bits
        x = (1.0f + 0.25f * ((lane + i) & 3)) * (float)(1 << ((lane >> 2) & 3)) * 0.125f;
        y = ((i & 1) ? -1.0f : 1.0f) * (1.0f + 0.25f * ((lane * 3 + i) & 3)) * (float)(1 << (i & 3)) * 0.25f;
      } else {
        x = 0.001f * (lane + i);
        y = 0.002f * (lane - i);
      }
      a[i] = (_Float16)x;
      b[i] = (_Float16)y;
      ab[i] = (__bf16)x;
      bb[i] = (__bf16)y;
    }
    for (int it = 0; it < iters; it++) {
#pragma unroll
      for (int j = 0; j < 8; j++) {
        if constexpr (KIND == 0 || KIND == 4)
          acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[j], 0, 0, 0);
        else
          acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab, bb, acc[j], 0, 0, 0);
      }
    }
  } else {
    const int base = 0x38383838 + lane;
    const v8i a = v8i{base, base + 1, base + 2, base + 3, base + 4, base + 5, base + 6, base + 7};
    const v8i b = v8i{base + 7, base + 6, base + 5, base + 4, base + 3, base + 2, base + 1, base};
    constexpr int fmt = KIND == 2 ? 0 : 4;  // 0: fp8 E4M3, 4: fp4 E2M1
    for (int it = 0; it < iters; it++) {
#pragma unroll
      for (int j = 0; j < 8; j++)
        acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[j], fmt, fmt, 0, 127, 0, 127);
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; j++)
#pragma unroll
    for (int r = 0; r < 16; r++) s += acc[j][r];
  if (flag) sink[blockIdx.x * 256 + threadIdx.x] = s;
}

__global__ void __launch_bounds__(256) read_probe(const uint4* __restrict__ p, int64_t n16, int flag,
                                                  uint32_t* sink) {
  uint32_t x = 0;
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 v0 = p[i], v1 = p[i + stride], v2 = p[i + 2 * stride], v3 = p[i + 3 * stride];
    x ^= v0.x ^ v0.y ^ v0.z ^ v0.w ^ v1.x ^ v1.y ^ v1.z ^ v1.w ^ v2.x ^ v2.y ^ v2.z ^ v2.w ^ v3.x ^ v3.y ^ v3.z ^
         v3.w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = p[i];
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (flag) sink[blockIdx.x * 256 + threadIdx.x] = x;
}

}  // namespace

int64_t probe_mfma_grid() { return 4 * (int64_t)device_cu_count(); }

hipError_t launch_probe_mfma(int kind, int iters, hipStream_t stream) {
  const unsigned grid = (unsigned)probe_mfma_grid();
  switch (kind) {
    case 0: mfma_probe<0><<<grid, 256, 0, stream>>>(iters, 0, nullptr); break;
    case 1: mfma_probe<1><<<grid, 256, 0, stream>>>(iters, 0, nullptr); break;
    case 2: mfma_probe<2><<<grid, 256, 0, stream>>>(iters, 0, nullptr); break;
    case 3: mfma_probe<3><<<grid, 256, 0, stream>>>(iters, 0, nullptr); break;
    case 4: mfma_probe<4><<<grid, 256, 0, stream>>>(iters, 0, nullptr); break;
    case 5: mfma_probe<5><<<grid, 256, 0, stream>>>(iters, 0, nullptr); break;
    case 6: mfma_probe<6><<<grid, 256, 0, stream>>>(iters, 0, nullptr); break;
    default: mfma_probe<7><<<grid, 256, 0, stream>>>(iters, 0, nullptr); break;
  }
  return hipGetLastError();
}

hipError_t launch_probe_read(const void* buf, int64_t bytes, hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  // four 16-byte loads per lane in flight; enough workgroups to cover every CU
  int64_t grid = (n16 + 4 * 256 - 1) / (4 * 256);
  const int64_t cap = 8 * (int64_t)device_cu_count();
  if (grid > cap) grid = cap;
  if (grid < 1) grid = 1;
  read_probe<<<(unsigned)grid, 256, 0, stream>>>(static_cast<const uint4*>(buf), n16, 0, nullptr);
  return hipGetLastError();
}

}  // namespace bsfp4

// Small-M GEMMs with NVFP4 weights (decode / small-batch shapes, HBM-bound):
//   NVFP4 W4A4:  D = bf16(alpha * dec(A) @ dec(B)^T)      (A, B NVFP4)
//   W4A16:       D = bf16(alpha * A @ dec(B)^T)           (A bf16, B NVFP4)
//
// These are the small-M rows of the pages' GEMM tables ("perf(gemm): optimize
// SM103 CuTe DSL mm_fp4 kernel", "Performance": M = 1..256 at N = 4096,
// K = 7168; "feat: sm100 cute_dsl w4a16 gemm", follow-up PR body: M = 1..128),
// where time is set by streaming the weights once.  A reviewer on the first
// page notes that narrow output tiles are what make the small-M case fast;
// here the narrowest tile is 16 output columns.
//
// Decomposition (one workgroup per 16 consecutive output columns n):
//   * the workgroup's waves split K into slices of 1024 elements; in a slice
//     lane l (row n0 + l%16, quarter g = l/16) owns 256 consecutive K values:
//     128 code bytes (eight 128-bit loads) and 16 scale bytes (one load), all
//     issued before any arithmetic so that a workgroup keeps its whole share of
//     the weight stream in flight;
//   * the activations for the same K values come from L2 (they are shared by
//     every workgroup);
//   * each 32-value step is one v_mfma_f32_16x16x32_{f16,bf16} with the
//     dequantised weights as the A operand (16 columns n) and the activations
//     as the B operand (16 rows m), so the K index of each lane's eight values
//     is the same on both sides;
//   * the per-wave partial tiles are summed in LDS in a fixed order (the result
//     is deterministic), multiplied by alpha and rounded once to bf16.
//
// Exactness: E2M1 x E4M3 products are exact in fp16 (W4A4: both operands) and
// in bf16 (W4A16 weights: at most 6 significant bits, range [2^-10, 2688]).
#include "device_common.h"
#include "launchers.h"

namespace bsfp4 {
namespace {

constexpr int kSlice = 1024;  // K values per wave per slice
constexpr int kLaneK = 256;   // K values per lane per slice

template <bool kAligned>
__device__ __forceinline__ uint4 load_scales16(const uint8_t* rowp, int64_t blk0, int64_t nblk) {
  // 16 scale bytes for blocks [blk0, blk0 + 16); blocks >= nblk read as 0.
  if (kAligned && blk0 + 16 <= nblk) return *reinterpret_cast<const uint4*>(rowp + blk0);
  uint32_t w[8];
  const uint16_t* p = reinterpret_cast<const uint16_t*>(rowp);
#pragma unroll
  for (int j = 0; j < 8; j++) w[j] = (blk0 + 2 * j < nblk) ? p[blk0 / 2 + j] : 0u;
  return make_uint4(w[0] | (w[1] << 16), w[2] | (w[3] << 16), w[4] | (w[5] << 16), w[6] | (w[7] << 16));
}

__device__ __forceinline__ void load_codes(uint4 (&c)[8], const uint8_t* rowp, int64_t byte0, int64_t nbytes) {
#pragma unroll
  for (int j = 0; j < 8; j++) {
    const int64_t b = byte0 + 16 * j;
    c[j] = (b < nbytes) ? *reinterpret_cast<const uint4*>(rowp + b) : make_uint4(0, 0, 0, 0);
  }
}

__device__ __forceinline__ uint32_t word_of(const uint4 (&c)[8], int w) {
  const uint4 v = c[w >> 2];
  const int s = w & 3;
  return s == 0 ? v.x : s == 1 ? v.y : s == 2 ? v.z : v.w;
}

__device__ __forceinline__ uint32_t byte_of(const uint4& v, int i) {
  const int s = i >> 2;
  const uint32_t w = s == 0 ? v.x : s == 1 ? v.y : s == 2 ? v.z : v.w;
  return (w >> (8 * (i & 3))) & 0xFFu;
}

// E4M3 byte -> fp16 (exact): the 7 magnitude bits at fp16 bit 7 give the value
// times 2^-8 for normal and subnormal codes; multiplying by 256 restores it.
__device__ __forceinline__ _Float16 e4m3_to_f16(uint32_t c) {
  const uint16_t bits = (uint16_t)((c & 0x7Fu) << 7);
  return __builtin_bit_cast(_Float16, bits) * (_Float16)256.0f;
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
  if (e == 0) return (float)m * 0.001953125f;
  return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

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

// Eight E2M1 values times an f32 scale -> eight bf16 (exact: <= 6 significant bits).
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
    // exact products: truncating to the upper 16 bits is the bf16 value
    o[j] = (__float_as_uint(f.x * s) >> 16) | (__float_as_uint(f.y * s) & 0xFFFF0000u);
  }
  return __builtin_bit_cast(v8bf, make_uint4(o[0], o[1], o[2], o[3]));
}

// AKIND 0: activations are NVFP4 (codes + E4M3 scales), fp16 MFMA.
// AKIND 1: activations are bf16, bf16 MFMA.
template <int AKIND, int MT, bool kAligned>
__global__ void __launch_bounds__(512)
    skinny_gemm(const void* __restrict__ Aptr, const uint8_t* __restrict__ SFA,
                const uint8_t* __restrict__ B, const uint8_t* __restrict__ SFB,
                const float* __restrict__ alpha_ptr, uint16_t* __restrict__ D, int M, int N, int64_t K) {
  __shared__ float red[8][MT][16][17];  // [wave][m tile][n][m], padded
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  const int n0 = blockIdx.x * 16;
  const int li = lane & 15;   // n row (weights) / m row (activations) inside the 16-tile
  const int g = lane >> 4;    // K quarter of the slice
  const int64_t kbytes = K / 2, kblk = K / 16;
  const uint8_t* brow = B + (int64_t)(n0 + li) * kbytes;
  const uint8_t* bsrow = SFB + (int64_t)(n0 + li) * kblk;

  v4f acc[MT];
#pragma unroll
  for (int t = 0; t < MT; t++) acc[t] = v4f{};

  const int64_t nslices = (K + kSlice - 1) / kSlice;
  for (int64_t sl = wave; sl < nslices; sl += nwaves) {
    const int64_t k0 = sl * kSlice + (int64_t)g * kLaneK;  // this lane's first K value
    uint4 bc[8];
    load_codes(bc, brow, k0 / 2, kbytes);
    const uint4 bs = load_scales16<kAligned>(bsrow, k0 / 16, kblk);

    if constexpr (AKIND == 0) {
      const uint8_t* A = static_cast<const uint8_t*>(Aptr);
#pragma unroll
      for (int t = 0; t < MT; t++) {
        const int m = t * 16 + li;
        uint4 ac[8];
        uint4 as = make_uint4(0, 0, 0, 0);
        if (m < M) {
          load_codes(ac, A + (int64_t)m * kbytes, k0 / 2, kbytes);
          as = load_scales16<kAligned>(SFA + (int64_t)m * kblk, k0 / 16, kblk);
        } else {
#pragma unroll
          for (int j = 0; j < 8; j++) ac[j] = make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int w = 0; w < 32; w++) {
          const v8h fb = dq8_f16(word_of(bc, w), e4m3_to_f16(byte_of(bs, w >> 1)));
          const v8h fa = dq8_f16(word_of(ac, w), e4m3_to_f16(byte_of(as, w >> 1)));
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fb, fa, acc[t], 0, 0, 0);
        }
      }
    } else {
      const uint16_t* A = static_cast<const uint16_t*>(Aptr);
#pragma unroll 4
      for (int w = 0; w < 32; w++) {
        const v8bf fb = dq8_bf16(word_of(bc, w), e4m3_to_f32(byte_of(bs, w >> 1)));
        const int64_t kk = k0 + 8 * w;
#pragma unroll
        for (int t = 0; t < MT; t++) {
          const int m = t * 16 + li;
          uint4 av = make_uint4(0, 0, 0, 0);
          if (m < M && kk < K) av = *reinterpret_cast<const uint4*>(A + (int64_t)m * K + kk);
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb, __builtin_bit_cast(v8bf, av), acc[t], 0, 0, 0);
        }
      }
    }
  }

  // acc[t][r] = partial D[m = t*16 + li][n = n0 + 4*g + r] of this wave
#pragma unroll
  for (int t = 0; t < MT; t++)
#pragma unroll
    for (int r = 0; r < 4; r++) red[wave][t][4 * g + r][li] = acc[t][r];
  __syncthreads();
  const float alpha = alpha_ptr ? alpha_ptr[0] : 1.0f;
  // thread -> (m, pair of n); fixed summation order over waves
  for (int idx = threadIdx.x; idx < MT * 16 * 8; idx += blockDim.x) {
    const int t = idx / 128, rem = idx % 128;
    const int mm = rem >> 3, np = (rem & 7) * 2;
    const int m = t * 16 + mm;
    if (m >= M) continue;
    float s0 = 0.0f, s1 = 0.0f;
    for (int w = 0; w < nwaves; w++) {
      s0 += red[w][t][np][mm];
      s1 += red[w][t][np + 1][mm];
    }
    *reinterpret_cast<uint32_t*>(D + (int64_t)m * N + n0 + np) = pack_bf16x2(alpha * s0, alpha * s1);
  }
}

template <int AKIND, int MT>
hipError_t launch_mt(const void* A, const uint8_t* SFA, const uint8_t* B, const uint8_t* SFB,
                     const float* alpha, uint16_t* D, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  const int64_t nslices = (K + kSlice - 1) / kSlice;
  const int waves = (int)(nslices < 8 ? nslices : 8);
  const dim3 grid((unsigned)(N / 16));
  if (K % 256 == 0)
    skinny_gemm<AKIND, MT, true><<<grid, 64 * waves, 0, stream>>>(A, SFA, B, SFB, alpha, D, (int)M, (int)N, K);
  else
    skinny_gemm<AKIND, MT, false><<<grid, 64 * waves, 0, stream>>>(A, SFA, B, SFB, alpha, D, (int)M, (int)N, K);
  return hipGetLastError();
}

template <int AKIND>
hipError_t launch_kind(const void* A, const uint8_t* SFA, const uint8_t* B, const uint8_t* SFB,
                       const float* alpha, uint16_t* D, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  if (M <= 16) return launch_mt<AKIND, 1>(A, SFA, B, SFB, alpha, D, M, N, K, stream);
  if (M <= 32) return launch_mt<AKIND, 2>(A, SFA, B, SFB, alpha, D, M, N, K, stream);
  return launch_mt<AKIND, 4>(A, SFA, B, SFB, alpha, D, M, N, K, stream);
}

}  // namespace

hipError_t launch_skinny_nvfp4(const uint8_t* A, const uint8_t* SFA, const uint8_t* B, const uint8_t* SFB,
                               const float* alpha, uint16_t* D, int64_t M, int64_t N, int64_t K,
                               hipStream_t stream) {
  return launch_kind<0>(A, SFA, B, SFB, alpha, D, M, N, K, stream);
}

hipError_t launch_skinny_w4a16(const uint16_t* A, const uint8_t* B, const uint8_t* SFB, const float* alpha,
                               uint16_t* D, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  return launch_kind<1>(A, nullptr, B, SFB, alpha, D, M, N, K, stream);
}

}  // namespace bsfp4

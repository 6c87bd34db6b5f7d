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
// Kernels (launch_kind picks the first that applies; the row kernel of
// gemm_w4a16.hip has already taken 17..64 W4A16 rows and 24..64 NVFP4 rows when
// K % 128 == 0):
//   * skinny_lds_few: at most four rows, K <= 8192 (also the fused quantise +
//     GEMM of nvfp4_quantize_gemm);
//   * skinny_lds: NVFP4 activations, up to 16 rows, K <= 8192;
//   * skinny_onepass: NVFP4 activations, up to 16 rows, K up to what its 8
//     waves cover;
//   * skinny_split: split-K form with one or two 16-row tiles (up to 32 rows),
//     and four tiles (33..64 rows) for bf16 activations, when the weights fit
//     32-bit buffer offsets;
//   * skinny_gemm: the original form described below, for 33..64 rows of
//     NVFP4 activations and for weights of 2^31 bytes or more (64-bit
//     addressing).
//
// skinny_gemm decomposition (one workgroup per 16 consecutive output columns n):
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
#include <cstdlib>

#include "device_common.h"
#include "launchers.h"
#include "lds_dma.h"
#include "quant_device.h"

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

// ---------------------------------------------------------------------------
// Split-K form for M <= 32 (one or two 16-row M tiles).  Work item = 64 output
// columns x a K range of KR = 128*NL values; the ranges of one column block are
// summed afterwards by splitk_reduce in range order (deterministic).
//   * every lane issues all of its weight loads for the range at once (NL
//     128-bit code loads and NL 2-byte scale loads, buffer loads that read zero
//     past K), four lanes covering 64 contiguous bytes of a weight row;
//   * meanwhile the workgroup writes the activations of the range into LDS as
//     fp16 (NVFP4 activations, dequantised once per workgroup) or bf16, so the
//     MFMA loop reads them with one ds_read_b128 per step;
//   * wave w owns output columns 16w..16w+15 of the block; lane (c, g) feeds
//     weight row c and the K values 128j + 32g + 8s (step s of load j) to
//     v_mfma_f32_16x16x32 as its A operand, the activations of the same K values
//     as B operand, so the lane ends with four consecutive columns of one row.
constexpr int kSkinnyCols = 64;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t skinny_rsrc(const void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

template <int AKIND, int MT, int NL>
__global__ void __launch_bounds__(256)
    skinny_split(const void* __restrict__ Aptr, const uint8_t* __restrict__ SFA, const uint8_t* __restrict__ B,
                 const uint8_t* __restrict__ SFB, const float* __restrict__ alpha_ptr, uint16_t* __restrict__ D,
                 int M, int N, int K, int ksplit, float* __restrict__ part) {
  constexpr int KR = 128 * NL;
  constexpr int kPitch = 2 * KR + 16;  // LDS bytes per activation row (odd number of 16-byte units)
  __shared__ __attribute__((aligned(16))) uint8_t act[MT * 16 * kPitch];
  constexpr uint32_t kOOB = 0x80000000u;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cb = blockIdx.x / ksplit, split = blockIdx.x % ksplit;
  const int n0 = cb * kSkinnyCols;
  const int k_lo = split * KR;
  const int k_hi = min(K, k_lo + KR);
  const int c = lane & 15, g = lane >> 4;
  // activation rows 8-15 of each 16-row tile hold their 64-byte K chunks pairwise
  // swapped (chunk ch at ch ^ 1), so the 16 lanes of one ds_read_b128 phase fall
  // on distinct banks
  const int swz = ((c >> 3) & 1) << 6;

  // ---- activation loads first (few, L2-resident): the per-wave memory queue
  // returns in order, so loads issued after the weight stream would wait for it
  constexpr int kItems = MT * 16 * (KR / 32);  // (row, 32-value chunk) items
  constexpr int kPer = (kItems + 255) / 256;
  uint4 aq[kPer][AKIND == 0 ? 1 : 4];
  uint32_t as2[kPer];
#pragma unroll
  for (int u = 0; u < kPer; u++) {
    const int it = tid + 256 * u;
    const int row = it / (KR / 32), ch = it % (KR / 32);
    const int k = k_lo + 32 * ch;
    const bool ok = it < kItems && row < M && k < k_hi;
    as2[u] = 0;
    if constexpr (AKIND == 0) {
      const uint8_t* A = static_cast<const uint8_t*>(Aptr);
      aq[u][0] = make_uint4(0, 0, 0, 0);
      if (ok) {
        aq[u][0] = *reinterpret_cast<const uint4*>(A + (int64_t)row * (K / 2) + k / 2);
        as2[u] = *reinterpret_cast<const uint16_t*>(SFA + (int64_t)row * (K / 16) + k / 16);
      }
    } else {
      const uint16_t* A = static_cast<const uint16_t*>(Aptr);
#pragma unroll
      for (int h = 0; h < 4; h++)
        aq[u][h] = ok ? *reinterpret_cast<const uint4*>(A + (int64_t)row * K + k + 8 * h) : make_uint4(0, 0, 0, 0);
    }
  }

  // ---- weight loads for the whole range (in flight while A is staged)
  const int n = n0 + 16 * wave + c;
  const __amdgpu_buffer_rsrc_t rq = skinny_rsrc(B, (int64_t)N * (K / 2));
  const __amdgpu_buffer_rsrc_t rs = skinny_rsrc(SFB, (int64_t)N * (K / 16));
  uint4 code[NL];
  uint32_t sc[NL];
#pragma unroll
  for (int j = 0; j < NL; j++) {
    const int k = k_lo + 128 * j + 32 * g;
    const bool ok = n < N && k < k_hi;
    const uint32_t oc = ok ? (uint32_t)((int64_t)n * (K / 2) + k / 2) : kOOB;
    const uint32_t os = ok ? (uint32_t)((int64_t)n * (K / 16) + k / 16) : kOOB;
    code[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rq, (int)oc, 0, 0));
    sc[j] = __builtin_amdgcn_raw_buffer_load_b16(rs, (int)os, 0, 0);
  }

  // ---- activations of the range -> LDS (rows >= M and K >= k_hi as zeros)
#pragma unroll
  for (int u = 0; u < kPer; u++) {
    const int it = tid + 256 * u;
    if (it >= kItems) break;
    const int row = it / (KR / 32), ch = it % (KR / 32);
    uint8_t* dst = act + row * kPitch + ((ch ^ ((row >> 3) & 1)) * 64);
    if constexpr (AKIND == 0) {
      const _Float16 s0 = e4m3_to_f16(as2[u] & 0xFFu), s1 = e4m3_to_f16(as2[u] >> 8);
      *reinterpret_cast<v8h*>(dst) = dq8_f16(aq[u][0].x, s0);
      *reinterpret_cast<v8h*>(dst + 16) = dq8_f16(aq[u][0].y, s0);
      *reinterpret_cast<v8h*>(dst + 32) = dq8_f16(aq[u][0].z, s1);
      *reinterpret_cast<v8h*>(dst + 48) = dq8_f16(aq[u][0].w, s1);
    } else {
#pragma unroll
      for (int h = 0; h < 4; h++) *reinterpret_cast<uint4*>(dst + 16 * h) = aq[u][h];
    }
  }
  __syncthreads();

  // ---- MFMA loop: load j, step s covers K values 128j + 32g + 8s .. +8 of the range
  v4f acc[MT];
#pragma unroll
  for (int t = 0; t < MT; t++) acc[t] = v4f{};
#pragma unroll
  for (int j = 0; j < NL; j++) {
#pragma unroll
    for (int s = 0; s < 4; s++) {
      const uint32_t word = s == 0 ? code[j].x : s == 1 ? code[j].y : s == 2 ? code[j].z : code[j].w;
      const uint32_t sbyte = (sc[j] >> (8 * (s >> 1))) & 0xFFu;
      const int koff = (2 * (128 * j + 32 * g + 8 * s)) ^ swz;
      if constexpr (AKIND == 0) {
        const v8h fb = dq8_f16(word, e4m3_to_f16(sbyte));
#pragma unroll
        for (int t = 0; t < MT; t++) {
          const v8h fa = *reinterpret_cast<const v8h*>(act + (t * 16 + c) * kPitch + koff);
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fb, fa, acc[t], 0, 0, 0);
        }
      } else {
        const v8bf fb = dq8_bf16(word, e4m3_to_f32(sbyte));
#pragma unroll
        for (int t = 0; t < MT; t++) {
          const v8bf fa = *reinterpret_cast<const v8bf*>(act + (t * 16 + c) * kPitch + koff);
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb, fa, acc[t], 0, 0, 0);
        }
      }
    }
  }

  // ---- lane holds D[m = 16t + c][n0 + 16*wave + 4g + r], r = 0..3
  const float alpha = alpha_ptr ? alpha_ptr[0] : 1.0f;
  const int ncol = n0 + 16 * wave + 4 * g;
#pragma unroll
  for (int t = 0; t < MT; t++) {
    const int m = t * 16 + c;
    if (m >= M || ncol >= N) continue;
    if (ksplit == 1) {
      *reinterpret_cast<uint2*>(D + (int64_t)m * N + ncol) =
          make_uint2(pack_bf16x2(alpha * acc[t][0], alpha * acc[t][1]), pack_bf16x2(alpha * acc[t][2], alpha * acc[t][3]));
    } else {
      *reinterpret_cast<float4*>(part + ((int64_t)split * M + m) * N + ncol) =
          make_float4(acc[t][0], acc[t][1], acc[t][2], acc[t][3]);
    }
  }
}

// ---------------------------------------------------------------------------
// Single-pass form for NVFP4 activations with M <= 16: one workgroup per 16
// output columns, its waves splitting K into ranges of 128*NL values.  Every
// lane loads both its weight row's codes/scales and the matching activation
// codes/scales for its whole range at once (the activations are L2-resident:
// every workgroup reads the same few rows), dequantises both operands in
// registers, and the waves' partial tiles are summed in LDS in wave order.  No
// second kernel and no workspace: for these sizes a split-K reduce launch
// costs more than the repeated activation dequantisation.
template <int NL>
__global__ void __launch_bounds__(512)
    skinny_onepass(const uint8_t* __restrict__ A, const uint8_t* __restrict__ SFA, const uint8_t* __restrict__ B,
                   const uint8_t* __restrict__ SFB, const float* __restrict__ alpha_ptr, uint16_t* __restrict__ D,
                   int M, int N, int K) {
  constexpr int KR = 128 * NL;
  constexpr uint32_t kOOB = 0x80000000u;
  __shared__ float red[8][16][17];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nwaves = blockDim.x >> 6;
  const int n0 = blockIdx.x * 16;
  const int c = lane & 15, g = lane >> 4;
  const int k_lo = wave * KR;
  const int n = n0 + c;
  const __amdgpu_buffer_rsrc_t rbq = skinny_rsrc(B, (int64_t)N * (K / 2));
  const __amdgpu_buffer_rsrc_t rbs = skinny_rsrc(SFB, (int64_t)N * (K / 16));
  const __amdgpu_buffer_rsrc_t raq = skinny_rsrc(A, (int64_t)M * (K / 2));
  const __amdgpu_buffer_rsrc_t ras = skinny_rsrc(SFA, (int64_t)M * (K / 16));
  uint4 ac[NL], bc[NL];
  uint32_t as[NL], bsc[NL];
  // activations first: the per-wave memory queue returns in order
#pragma unroll
  for (int j = 0; j < NL; j++) {
    const int k = k_lo + 128 * j + 32 * g;
    const bool ok = c < M && k < K;
    const uint32_t oc = ok ? (uint32_t)(c * (K / 2) + k / 2) : kOOB;
    const uint32_t os = ok ? (uint32_t)(c * (K / 16) + k / 16) : kOOB;
    ac[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(raq, (int)oc, 0, 0));
    as[j] = __builtin_amdgcn_raw_buffer_load_b16(ras, (int)os, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < NL; j++) {
    const int k = k_lo + 128 * j + 32 * g;
    const bool ok = n < N && k < K;
    const uint32_t oc = ok ? (uint32_t)((int64_t)n * (K / 2) + k / 2) : kOOB;
    const uint32_t os = ok ? (uint32_t)((int64_t)n * (K / 16) + k / 16) : kOOB;
    bc[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rbq, (int)oc, 0, 0));
    bsc[j] = __builtin_amdgcn_raw_buffer_load_b16(rbs, (int)os, 0, 0);
  }
  v4f acc = v4f{};
#pragma unroll
  for (int j = 0; j < NL; j++) {
#pragma unroll
    for (int s = 0; s < 4; s++) {
      const uint32_t wb = s == 0 ? bc[j].x : s == 1 ? bc[j].y : s == 2 ? bc[j].z : bc[j].w;
      const uint32_t wa = s == 0 ? ac[j].x : s == 1 ? ac[j].y : s == 2 ? ac[j].z : ac[j].w;
      const v8h fb = dq8_f16(wb, e4m3_to_f16((bsc[j] >> (8 * (s >> 1))) & 0xFFu));
      const v8h fa = dq8_f16(wa, e4m3_to_f16((as[j] >> (8 * (s >> 1))) & 0xFFu));
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(fb, fa, acc, 0, 0, 0);
    }
  }
  // acc[r] = partial D[m = c][n0 + 4g + r] of this wave's K range
#pragma unroll
  for (int r = 0; r < 4; r++) red[wave][4 * g + r][c] = acc[r];
  __syncthreads();
  for (int idx = tid; idx < 16 * 8; idx += blockDim.x) {  // (row, column pair); a single wave loops
    const int m = idx >> 3, np = (idx & 7) * 2;
    if (m < M) {
      float s0 = 0.0f, s1 = 0.0f;
      for (int w = 0; w < nwaves; w++) {
        s0 += red[w][np][m];
        s1 += red[w][np + 1][m];
      }
      const float alpha = alpha_ptr ? alpha_ptr[0] : 1.0f;
      *reinterpret_cast<uint32_t*>(D + (int64_t)m * N + n0 + np) = pack_bf16x2(alpha * s0, alpha * s1);
    }
  }
}

// ---------------------------------------------------------------------------
// LDS-staged single-pass form for NVFP4 activations, M <= 16, K <= 8192: one
// workgroup per 16 output columns, nw <= 15 waves each owning UW units of 128
// K values (UW = 4 and 14 waves at K = 7168).  Measured on the GPU, the
// per-lane register loads of the forms above spend most of their time in the
// vector memory pipeline (each 16-lane quarter of a load touches 16 rows, and
// 2-byte scale loads cost as much as code loads), so here every operand
// reaches LDS through direct-to-LDS DMA:
//   * scales: when a row's scale bytes are a multiple of 16 (K % 256 == 0),
//     each wave copies the 16 x 64 bytes of its own K range for the weight and
//     for the activation rows (one instruction each) and needs no other
//     wave's data, so no barrier precedes the dequantisation: a wave starts as
//     soon as its own loads land (a workgroup barrier there made every wave
//     wait for the slowest one's whole issue, measured 10.3 -> 9.3 us at
//     16 x 4096 x 7168 cold).  Otherwise the workgroup's 16 weight rows of
//     scales, one contiguous 16 x K/16-byte block in memory (row-major
//     [N, K/16]), and likewise the 16 activation rows are copied KB by KB by
//     the waves and one barrier makes them visible to all;
//   * codes: weight and activation units move in pairs of 8 rows x 128 B (see
//     below);
//   * the activations are issued first (L2-resident) and dequantised into
//     registers while the weight stream is still in flight; then each weight
//     unit is consumed as soon as its own DMA has landed (s_waitcnt vmcnt);
//     more, shorter waves (4 units each instead of 8) shorten the dequantise
//     and MFMA tail of the wave whose loads are served last (9.3 -> 9.0 us);
//   * partial 16 x 16 tiles are summed in LDS in wave order (deterministic),
//     multiplied by alpha and rounded once to bf16.
// Lanes past the problem (rows >= M, K >= K) read zeros; scale bytes past a
// row's end only ever multiply zero codes.
constexpr int kLdsMaxWaves = 8;  // waves of the few-row form

// Waves of the M <= 16 LDS form with UW units per wave: as many as fit in the
// 160 KB of LDS (2 + 2 UW KB per wave), at most 15.
__host__ __device__ constexpr int lds_waves(int uw) { return 160 / (2 + 2 * uw) < 15 ? 160 / (2 + 2 * uw) : 15; }

// Code units of 128 K values are moved in pairs: one DMA instruction carries 8
// rows x 128 B (a pair of units of 8 rows: whole cache lines; 16 rows x 64 B
// per instruction, half lines, measured slower), so a pair of units of 16 rows
// is two instructions into LDS laid out [pair][row][128 B].  16-byte piece p
// (0..7) of row r sits at position p ^ (r & 7), so the 8 lanes of a 128-bit LDS
// read (rows c .. c+7, one piece each) hit distinct banks.
// LDS byte offset of unit i's piece g (0..3) of row c inside a wave's region:
__device__ __forceinline__ int pair_rd(int i, int c, int g) {
  return 2048 * (i >> 1) + c * 128 + ((((i & 1) * 4 + g) ^ (c & 7)) * 16);
}

// Issue the UW/2 unit pairs of 16 rows starting at global byte offset row0_off
// (row r at row0_off + r * row_bytes), K values [k_lo, k_lo + 128 UW) of each
// row; rows >= nrows and K beyond K read as zero.  dst: the wave's region.
template <int UW>
__device__ __forceinline__ void issue_pairs(v4u32 rsrc, uint32_t row0_off, uint32_t row_bytes, int nrows, int k_lo,
                                            int K, const uint8_t* dst, int lane) {
  static_assert(UW % 2 == 0, "units come in pairs");
#pragma unroll
  for (int u = 0; u < UW / 2; u++) {
#pragma unroll
    for (int h = 0; h < 2; h++) {
      const int r = h * 8 + (lane >> 3);
      const int lp = (lane & 7) ^ (r & 7);  // logical piece landing at position lane & 7
      const bool ok = r < nrows && k_lo + 256 * u + 32 * lp < K;
      buf_lds16(rsrc, ok ? row0_off + (uint32_t)r * row_bytes + (uint32_t)(k_lo / 2 + 128 * u + 16 * lp) : kBufOOB, 0,
                (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_offset(dst + 2048 * u + 1024 * h)));
    }
  }
}

template <int UW>
__global__ void __launch_bounds__(1024)
    skinny_lds(const uint8_t* __restrict__ A, const uint8_t* __restrict__ SFA, const uint8_t* __restrict__ B,
               const uint8_t* __restrict__ SFB, const float* __restrict__ alpha_ptr, uint16_t* __restrict__ D,
               int M, int N, int K) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[(2 + 2 * UW) * lds_waves(UW) * 1024];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nwaves = blockDim.x >> 6;
  const int n0 = blockIdx.x * 16;
  const int k_lo = wave * (UW * 128);
  const int kb16 = K / 16;  // scale bytes per row
  uint8_t* const lsb = smem;                        // nwaves KB: weight scales, rows n0..n0+15
  uint8_t* const lsa = smem + nwaves * 1024;        // nwaves KB: activation scales, rows 0..15
  uint8_t* const lbq = smem + 2 * nwaves * 1024 + wave * (2 * UW * 1024);  // UW KB of weight codes
  uint8_t* const laq = lbq + UW * 1024;                                    // UW KB of activation codes
  const v4u32 rbq = make_rsrc4(B, (int64_t)N * (K / 2));
  const v4u32 rbs = make_rsrc4(SFB, (int64_t)N * kb16);
  const v4u32 raq = make_rsrc4(A, (int64_t)M * (K / 2));
  const v4u32 ras = make_rsrc4(SFA, (int64_t)M * kb16);
  const bool own_scales = (kb16 % 16) == 0;  // 16-byte aligned pieces of every row's scale bytes
  if (own_scales) {
    // this wave's K range [k_lo, k_lo + 128 UW): 8 UW scale bytes of each of 16 rows, lane = (row, 16-byte piece);
    // the pieces past the range belong to the next wave and are never read here
    const int r = lane >> 2, pc = k_lo / 16 + 16 * (lane & 3);
    buf_lds16(rbs, pc < kb16 ? (uint32_t)((n0 + r) * kb16 + pc) : kBufOOB, 0,
              (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_offset(lsb + wave * 1024)));
    buf_lds16(ras, (r < M && pc < kb16) ? (uint32_t)(r * kb16 + pc) : kBufOOB, 0,
              (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_offset(lsa + wave * 1024)));
  } else {
    const int off = wave * 1024 + lane * 16;  // byte of the 16 x K/16 scale block
    buf_lds16(rbs, off < 16 * kb16 ? (uint32_t)(n0 * kb16 + off) : kBufOOB, 0,
              (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_offset(lsb + wave * 1024)));
    buf_lds16(ras, off < M * kb16 ? (uint32_t)off : kBufOOB, 0,
              (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_offset(lsa + wave * 1024)));
  }
  issue_pairs<UW>(raq, 0u, (uint32_t)(K / 2), M, k_lo, K, laq, lane);
  issue_pairs<UW>(rbq, (uint32_t)(n0 * (K / 2)), (uint32_t)(K / 2), 16, k_lo, K, lbq, lane);

  // MFMA lane (c, g): row c, K values 128i + 32g + 8s (s = word of the piece)
  const int c = lane & 15, g = lane >> 4;
  wait_vmcnt<UW>();  // scales and activations have landed; only weight units may be in flight
  if (!own_scales) __builtin_amdgcn_s_barrier();  // the scale block was copied by all waves
  const uint8_t* sbrow = own_scales ? lsb + wave * 1024 + c * 64 + 2 * g : lsb + c * kb16 + k_lo / 16 + 2 * g;
  const uint8_t* sarow = own_scales ? lsa + wave * 1024 + c * 64 + 2 * g : lsa + c * kb16 + k_lo / 16 + 2 * g;
  // two E4M3 scale bytes -> two fp16 values (exact): magnitude bits at fp16 bit 7, times 2^8
  auto scales2 = [](uint32_t s) {
    return __builtin_bit_cast(v2h, ((s & 0x7Fu) << 7) | ((s & 0x7F00u) << 15)) *
           v2h{(_Float16)256.0f, (_Float16)256.0f};
  };
  v8h fa[UW][4];
#pragma unroll
  for (int i = 0; i < UW; i++) {
    const uint4 w = *reinterpret_cast<const uint4*>(laq + pair_rd(i, c, g));
    const v2h s = scales2(*reinterpret_cast<const uint16_t*>(sarow + 8 * i));
    fa[i][0] = dq8_f16(w.x, s[0]);
    fa[i][1] = dq8_f16(w.y, s[0]);
    fa[i][2] = dq8_f16(w.z, s[1]);
    fa[i][3] = dq8_f16(w.w, s[1]);
    // keep this dequantisation ahead of the weight waits
    asm volatile("" : "+v"(fa[i][0]), "+v"(fa[i][1]), "+v"(fa[i][2]), "+v"(fa[i][3]));
  }
  v4f acc = v4f{};
#pragma unroll
  for (int i = 0; i < UW; i++) {
    if ((i & 1) == 0) wait_vmcnt_upto(UW - 2 - i);  // the weight pair of unit i has landed
    const uint4 w = *reinterpret_cast<const uint4*>(lbq + pair_rd(i, c, g));
    const v2h s = scales2(*reinterpret_cast<const uint16_t*>(sbrow + 8 * i));
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(dq8_f16(w.x, s[0]), fa[i][0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(dq8_f16(w.y, s[0]), fa[i][1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(dq8_f16(w.z, s[1]), fa[i][2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(dq8_f16(w.w, s[1]), fa[i][3], acc, 0, 0, 0);
    asm volatile("" : "+v"(acc));  // unit i is done before the next unit's wait
  }
  // acc[j] = partial D[m = c][n0 + 4g + j]; each wave's tile goes to its own code region
  float* red = reinterpret_cast<float*>(lbq);
#pragma unroll
  for (int j = 0; j < 4; j++) red[(4 * g + j) * 17 + c] = acc[j];
  __syncthreads();
  const float alpha = alpha_ptr ? alpha_ptr[0] : 1.0f;
  for (int idx = tid; idx < 128; idx += blockDim.x) {  // (row, column pair), waves summed in order
    const int m = idx >> 3, np = (idx & 7) * 2;
    if (m >= M) continue;
    float s0 = 0.0f, s1 = 0.0f;
    for (int w = 0; w < nwaves; w++) {
      const float* rw = reinterpret_cast<const float*>(smem + 2 * nwaves * 1024 + w * (2 * UW * 1024));
      s0 += rw[np * 17 + m];
      s1 += rw[(np + 1) * 17 + m];
    }
    *reinterpret_cast<uint32_t*>(D + (int64_t)m * N + n0 + np) = pack_bf16x2(alpha * s0, alpha * s1);
  }
}

// ---------------------------------------------------------------------------
// LDS-staged single-pass form for at most four activation rows (decode
// shapes), NVFP4 (AKIND 0) or bf16 (AKIND 1) activations, K <= 8192; AKIND 2
// is the fused quantise + GEMM: bf16 rows quantised to NVFP4 with the global
// scale gs inside the workgroup; AKIND 3 (NVFP4, one or two rows) runs the
// raw E2M1 codes on the scaled FP4 MFMA and applies the E4M3 block scales to
// the exact per-block dot products (see the main loop).  The
// weights move exactly as in skinny_lds.  The activation rows, being few, are
// copied whole into LDS once per workgroup (one contiguous block: rows are
// contiguous in memory) and, for NVFP4, dequantised there once to fp16 by all
// threads; the MFMA then reads its activation operand from LDS (lanes of rows
// >= M feed zeros), so the per-wave VALU work is the weight dequantisation
// alone instead of weights plus 16 mostly-empty activation rows.
constexpr int kFewRows = 4;

template <int AKIND, int UW>
__global__ void __launch_bounds__(512)
    skinny_lds_few(const void* __restrict__ Aptr, const uint8_t* __restrict__ SFA, const uint8_t* __restrict__ B,
                   const uint8_t* __restrict__ SFB, const float* __restrict__ alpha_ptr, uint16_t* __restrict__ D,
                   int M, int N, int K, const float* __restrict__ gs_ptr = nullptr) {
  constexpr int kMaxK = 1024 * UW;  // nw <= 8 waves of UW units of 128 values
  constexpr int kBScale = 8 * 1024;                                   // 16 x K/16 weight scale block
  constexpr int kBCodes = kLdsMaxWaves * UW * 1024;                   // per-wave [unit][row][64 B]
  constexpr int kAVals = kFewRows * kMaxK * 2;                        // fp16 / bf16 activation rows
  constexpr bool kFp4A = AKIND == 0 || AKIND == 3;                   // NVFP4 activations
  constexpr int kACodes = kFp4A ? kFewRows * kMaxK / 2 : 0;           // NVFP4 codes before dequantisation
  constexpr int kAScales = kFp4A ? ((kFewRows * kMaxK / 16 + 1023) / 1024) * 1024 : 0;
  static_assert(AKIND != 3 || (kMaxK / 16) * 64 + kFewRows * (kMaxK / 16) * 4 <= kAVals, "scale tables fit");
  __shared__ __attribute__((aligned(16))) uint8_t smem[kBScale + kBCodes + kAVals + kACodes + kAScales];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nwaves = blockDim.x >> 6;
  const int n0 = blockIdx.x * 16;
  const int k_lo = wave * (UW * 128);
  const int kb16 = K / 16;
  uint8_t* const lsb = smem;
  uint8_t* const lbq = smem + kBScale + wave * (UW * 1024);
  uint8_t* const lav = smem + kBScale + kBCodes;  // activation values, row m at m * 2K bytes
  uint8_t* const laq = lav + kAVals;              // NVFP4 activation codes [M][K/2]
  uint8_t* const las = laq + kACodes;             // NVFP4 activation scales [M][K/16]
  const v4u32 rbq = make_rsrc4(B, (int64_t)N * (K / 2));
  const v4u32 rbs = make_rsrc4(SFB, (int64_t)N * kb16);
  auto lds_u = [](const uint8_t* p) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_offset(p)); };

  // ---- weight scales (one 1 KB piece per wave) and the activation block(s),
  // pieces spread over the waves; all of them are issued before the weight
  // units, so waiting for "at most UW outstanding" covers them whatever their count
  {
    const int off = wave * 1024 + lane * 16;
    buf_lds16(rbs, off < 16 * kb16 ? (uint32_t)(n0 * kb16 + off) : kBufOOB, 0, lds_u(lsb + wave * 1024));
  }
  if constexpr (kFp4A) {
    const v4u32 raq = make_rsrc4(Aptr, (int64_t)M * (K / 2));
    const v4u32 ras = make_rsrc4(SFA, (int64_t)M * kb16);
    const int qpieces = (M * (K / 2) + 1023) / 1024, spieces = (M * kb16 + 1023) / 1024;
    for (int pc = wave; pc < qpieces + spieces; pc += nwaves) {  // codes first, then scales
      if (pc < qpieces) {
        const int off = pc * 1024 + lane * 16;
        buf_lds16(raq, off < M * (K / 2) ? (uint32_t)off : kBufOOB, 0, lds_u(laq + pc * 1024));
      } else {
        const int off = (pc - qpieces) * 1024 + lane * 16;
        buf_lds16(ras, off < M * kb16 ? (uint32_t)off : kBufOOB, 0, lds_u(las + (pc - qpieces) * 1024));
      }
    }
  } else {
    const v4u32 ra = make_rsrc4(Aptr, (int64_t)M * K * 2);
    const int apieces = (M * K * 2 + 1023) / 1024;
    for (int pc = wave; pc < apieces; pc += nwaves) {
      const int off = pc * 1024 + lane * 16;
      buf_lds16(ra, off < M * K * 2 ? (uint32_t)off : kBufOOB, 0, lds_u(lav + pc * 1024));
    }
  }
  // ---- weight units
  issue_pairs<UW>(rbq, (uint32_t)(n0 * (K / 2)), (uint32_t)(K / 2), 16, k_lo, K, lbq, lane);
  wait_vmcnt<UW>();  // activations and scales have landed
  __builtin_amdgcn_s_barrier();
  if constexpr (AKIND == 0) {  // dequantise the activation rows once: 8 values per item
    for (int it = tid; it < M * (K / 8); it += blockDim.x) {
      const int m = it / (K / 8), w = it - m * (K / 8);
      const uint32_t word = *reinterpret_cast<const uint32_t*>(laq + m * (K / 2) + 4 * w);
      const uint32_t sc = las[m * kb16 + (w >> 1)];
      *reinterpret_cast<v8h*>(lav + m * (2 * K) + 16 * w) = dq8_f16(word, e4m3_to_f16(sc));
    }
    __syncthreads();
  }
  if constexpr (AKIND == 2) {
    // Fused quantiser: each 16-value block of the bf16 rows (32 contiguous LDS
    // bytes; the rows are contiguous) goes through the NVFP4 quantiser's
    // binary32 steps with gs -- s = fl32(fl32(amax/6)*gs) to E4M3 (RNE,
    // saturating), inv = fl32(gs/dec(s)), codes = E2M1 RNE of fl32(v*inv) --
    // and is replaced in place by the exact fp16 values code * dec(s), i.e.
    // what the AKIND 0 path computes from fp4_quantize's output.
    const float gs = gs_ptr[0];
    for (int it = tid; it < M * kb16; it += blockDim.x) {
      uint8_t* blk = lav + 32 * it;
      const uint4 lo = *reinterpret_cast<const uint4*>(blk), hi = *reinterpret_cast<const uint4*>(blk + 16);
      const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      float v[16];
      float amax = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; j++) {
        v[2 * j] = bf16_bits_to_float(w[j] & 0xFFFFu);
        v[2 * j + 1] = bf16_bits_to_float(w[j] >> 16);
        amax = fmaxf(amax, fmaxf(fabsf(v[2 * j]), fabsf(v[2 * j + 1])));
      }
      const uint32_t scode = e4m3_rne_satfinite((amax / 6.0f) * gs);
      const float sdec = e4m3_decode(scode);
      const float inv = (sdec == 0.0f) ? 0.0f : gs / sdec;
      uint32_t q0 = 0, q1 = 0;
#pragma unroll
      for (int t = 0; t < 4; t++) {
        q0 = e2m1x2_f32(q0, v[2 * t] * inv, v[2 * t + 1] * inv, t);
        q1 = e2m1x2_f32(q1, v[8 + 2 * t] * inv, v[8 + 2 * t + 1] * inv, t);
      }
      const _Float16 sh = e4m3_to_f16(scode);
      *reinterpret_cast<v8h*>(blk) = dq8_f16(q0, sh);
      *reinterpret_cast<v8h*>(blk + 16) = dq8_f16(q1, sh);
    }
    __syncthreads();
  }

  // AKIND 3: scale tables in binary32 (E4M3 decoded exactly): weights as
  // [block][16 columns], activations as [row][block]
  float* const tsb = reinterpret_cast<float*>(lav);
  float* const tsa = tsb + (kMaxK / 16) * 16;
  if constexpr (AKIND == 3) {
    for (int it = tid; it < 16 * kb16; it += blockDim.x) {
      const int b = it >> 4, n = it & 15;
      tsb[it] = e4m3_to_f32(lsb[n * kb16 + b]);
    }
    for (int it = tid; it < M * kb16; it += blockDim.x) {
      const int m = it / kb16, b = it - m * kb16;
      tsa[m * (kMaxK / 16) + b] = e4m3_to_f32(las[m * kb16 + b]);
    }
    __syncthreads();
  }

  const int c = lane & 15, g = lane >> 4;
  const uint8_t* sbrow = lsb + c * kb16 + k_lo / 16 + 2 * g;
  const uint8_t* arow = lav + c * (2 * K) + 2 * (k_lo + 32 * g);
  v4f acc = v4f{};
#pragma unroll
  for (int i = 0; i < UW; i++) {
    if ((i & 1) == 0) wait_vmcnt_upto(UW - 2 - i);  // the weight pair of unit i has landed
    const uint4 w = *reinterpret_cast<const uint4*>(lbq + pair_rd(i, c, g));
    if constexpr (AKIND == 3) {
      // Re-blocked onto the scaled FP4 MFMA with unit scales: the second
      // operand is block-diagonal -- its row c holds activation row c/8's
      // codes of block c%8 of this 128-value unit and zeros elsewhere -- so
      // the MFMA yields the per-block dot products of raw E2M1 codes (exact),
      // and each is scaled by dec(sA)*dec(sB) (exact) before the FP32 sum.
      const int m = c >> 3, jb = c & 7;
      const int k_unit = k_lo + 128 * i;
      const bool live = m < M && (jb >> 1) == g && k_unit + 32 * g < K;
      uint2 ac = make_uint2(0, 0);
      if (live) ac = *reinterpret_cast<const uint2*>(laq + m * (K / 2) + k_unit / 2 + 8 * jb);
      const v8i fy = (jb & 1) ? v8i{0, 0, (int)ac.x, (int)ac.y, 0, 0, 0, 0}
                              : v8i{(int)ac.x, (int)ac.y, 0, 0, 0, 0, 0, 0};
      const v8i fx = v8i{(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
      v4f d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fx, fy, v4f{0, 0, 0, 0}, 4, 4, 0, 127, 0, 127);
      // The MFMA reads every lane's operands, so it must run with all lanes
      // active: the pin keeps the compiler from sinking it into the
      // lane-dependent code below, which is branch-free (selects) for the same
      // reason.  Table reads stay inside the tables (m <= 1, b < kMaxK/16).
      asm volatile("" : "+v"(d));
      const int b = k_unit / 16 + jb;  // this lane's block (its output column c)
      const bool use = m < M && b < kb16;
      const float sa = tsa[m * (kMaxK / 16) + b];
      const float4 sb4 = *reinterpret_cast<const float4*>(tsb + b * 16 + 4 * g);
      acc[0] += (use ? sa * sb4.x : 0.0f) * d[0];
      acc[1] += (use ? sa * sb4.y : 0.0f) * d[1];
      acc[2] += (use ? sa * sb4.z : 0.0f) * d[2];
      acc[3] += (use ? sa * sb4.w : 0.0f) * d[3];
      asm volatile("" : "+v"(acc));
      continue;
    }
    const uint32_t sb = *reinterpret_cast<const uint16_t*>(sbrow + 8 * i);
    uint4 av[4] = {};
    if (c < M && k_lo + 128 * i + 32 * g < K) {
#pragma unroll
      for (int q = 0; q < 4; q++) av[q] = *reinterpret_cast<const uint4*>(arow + 256 * i + 16 * q);
    }
    if constexpr (AKIND != 1) {  // fp16 activations (NVFP4 or fused-quantised)
      const v2h s = __builtin_bit_cast(v2h, ((sb & 0x7Fu) << 7) | ((sb & 0x7F00u) << 15)) *
                    v2h{(_Float16)256.0f, (_Float16)256.0f};
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(dq8_f16(w.x, s[0]), __builtin_bit_cast(v8h, av[0]), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(dq8_f16(w.y, s[0]), __builtin_bit_cast(v8h, av[1]), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(dq8_f16(w.z, s[1]), __builtin_bit_cast(v8h, av[2]), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(dq8_f16(w.w, s[1]), __builtin_bit_cast(v8h, av[3]), acc, 0, 0, 0);
    } else {
      const float s0 = e4m3_to_f32(sb & 0xFFu), s1 = e4m3_to_f32(sb >> 8);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dq8_bf16(w.x, s0), __builtin_bit_cast(v8bf, av[0]), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dq8_bf16(w.y, s0), __builtin_bit_cast(v8bf, av[1]), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dq8_bf16(w.z, s1), __builtin_bit_cast(v8bf, av[2]), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dq8_bf16(w.w, s1), __builtin_bit_cast(v8bf, av[3]), acc, 0, 0, 0);
    }
    asm volatile("" : "+v"(acc));  // unit i is done before the next unit's wait
  }
  if constexpr (AKIND == 3) {
    // sum the 8 blocks (lanes c = 8m .. 8m+7) into lane 8m, which then holds
    // column m of rows 4g .. 4g+3, like the other forms' lane (g, c = m)
#pragma unroll
    for (int o = 1; o < 8; o <<= 1)
#pragma unroll
      for (int j = 0; j < 4; j++) acc[j] += __shfl_xor(acc[j], o, 64);
  }
  float* red = reinterpret_cast<float*>(lbq);  // 16 x 16 floats: exactly the smallest (1 KB) region
#pragma unroll
  for (int j = 0; j < 4; j++) {
    if constexpr (AKIND == 3) {
      if ((c & 7) == 0) red[(4 * g + j) * 16 + (c >> 3)] = acc[j];
    } else {
      red[(4 * g + j) * 16 + c] = acc[j];
    }
  }
  __syncthreads();
  const float alpha = alpha_ptr ? alpha_ptr[0] : 1.0f;
  for (int idx = tid; idx < kFewRows * 8; idx += blockDim.x) {
    const int m = idx >> 3, np = (idx & 7) * 2;
    if (m >= M) continue;
    float s0 = 0.0f, s1 = 0.0f;
    for (int w = 0; w < nwaves; w++) {
      const float* rw = reinterpret_cast<const float*>(smem + kBScale + w * (UW * 1024));
      s0 += rw[np * 16 + m];
      s1 += rw[(np + 1) * 16 + m];
    }
    *reinterpret_cast<uint32_t*>(D + (int64_t)m * N + n0 + np) = pack_bf16x2(alpha * s0, alpha * s1);
  }
}

// NL for the single-pass form (<= 8 waves of 128*NL values), 0 if K is too long.
int onepass_nl(int64_t K) {
  const int64_t kb = (K + 127) / 128;
  const int opts[6] = {1, 2, 4, 7, 8, 14};
  for (int o : opts)
    if ((kb + o - 1) / o <= 8) return o;
  return 0;
}

// Loads per lane per work item and the split count for an M <= 32 problem:
// about two work items per CU, at most 16 loads (2048 K values) per lane.
struct SkinnyPlan {
  int nl, ksplit;
};
int env_skinny_per_cu() {
  const char* e = getenv("BSFP4_SKINNY_PER_CU");
  return e ? atoi(e) : 1;
}
SkinnyPlan skinny_plan(int64_t N, int64_t K, int cus, int mt) {
  const int64_t blocks = (N + kSkinnyCols - 1) / kSkinnyCols;
  const int64_t kb = (K + 127) / 128;  // 128-value blocks
  const int per_cu = env_skinny_per_cu();
  int64_t ks = (per_cu * cus + blocks - 1) / blocks;
  if (ks < 1) ks = 1;
  if (ks > kb) ks = kb;
  int64_t nl = (kb + ks - 1) / ks;
  // the activation tile (16*mt rows x 128*nl values, 2 bytes each) must fit in LDS
  const int max_nl = mt >= 4 ? 8 : 16;
  const int opts[5] = {2, 4, 8, 14, 16};
  int pick = max_nl;
  for (int o : opts)
    if (o >= nl && o <= max_nl) { pick = o; break; }
  const int64_t ksplit = (kb + pick - 1) / pick;
  return SkinnyPlan{pick, (int)ksplit};
}


template <int AKIND, int MT, int NL>
hipError_t launch_split_nl(const void* A, const uint8_t* SFA, const uint8_t* B, const uint8_t* SFB,
                           const float* alpha, uint16_t* D, int64_t M, int64_t N, int64_t K, int ksplit,
                           float* part, hipStream_t stream) {
  const unsigned grid = (unsigned)(((N + kSkinnyCols - 1) / kSkinnyCols) * ksplit);
  skinny_split<AKIND, MT, NL><<<grid, 256, 0, stream>>>(A, SFA, B, SFB, alpha, D, (int)M, (int)N, (int)K, ksplit,
                                                        part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || ksplit == 1) return e;
  return launch_splitk_reduce(part, ksplit, alpha, D, M * N, stream);
}

template <int AKIND, int MT>
hipError_t launch_split(const void* A, const uint8_t* SFA, const uint8_t* B, const uint8_t* SFB,
                        const float* alpha, uint16_t* D, int64_t M, int64_t N, int64_t K, float* part,
                        hipStream_t stream) {
  const SkinnyPlan pl = skinny_plan(N, K, device_cu_count(), MT);
  switch (pl.nl) {
    case 2: return launch_split_nl<AKIND, MT, 2>(A, SFA, B, SFB, alpha, D, M, N, K, pl.ksplit, part, stream);
    case 4: return launch_split_nl<AKIND, MT, 4>(A, SFA, B, SFB, alpha, D, M, N, K, pl.ksplit, part, stream);
    case 8: return launch_split_nl<AKIND, MT, 8>(A, SFA, B, SFB, alpha, D, M, N, K, pl.ksplit, part, stream);
    default:
      if constexpr (MT < 4) {
        if (pl.nl == 14)
          return launch_split_nl<AKIND, MT, 14>(A, SFA, B, SFB, alpha, D, M, N, K, pl.ksplit, part, stream);
        return launch_split_nl<AKIND, MT, 16>(A, SFA, B, SFB, alpha, D, M, N, K, pl.ksplit, part, stream);
      }
      return hipErrorInvalidValue;  // not planned: nl <= 8 for four M tiles
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

template <int NL>
hipError_t launch_onepass_nl(const uint8_t* A, const uint8_t* SFA, const uint8_t* B, const uint8_t* SFB,
                             const float* alpha, uint16_t* D, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  const int waves = (int)(((K + 127) / 128 + NL - 1) / NL);
  skinny_onepass<NL><<<(unsigned)(N / 16), 64 * waves, 0, stream>>>(A, SFA, B, SFB, alpha, D, (int)M, (int)N,
                                                                     (int)K);
  return hipGetLastError();
}

hipError_t launch_onepass(const uint8_t* A, const uint8_t* SFA, const uint8_t* B, const uint8_t* SFB,
                          const float* alpha, uint16_t* D, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  switch (onepass_nl(K)) {
    case 1: return launch_onepass_nl<1>(A, SFA, B, SFB, alpha, D, M, N, K, stream);
    case 2: return launch_onepass_nl<2>(A, SFA, B, SFB, alpha, D, M, N, K, stream);
    case 4: return launch_onepass_nl<4>(A, SFA, B, SFB, alpha, D, M, N, K, stream);
    case 7: return launch_onepass_nl<7>(A, SFA, B, SFB, alpha, D, M, N, K, stream);
    case 8: return launch_onepass_nl<8>(A, SFA, B, SFB, alpha, D, M, N, K, stream);
    default: return launch_onepass_nl<14>(A, SFA, B, SFB, alpha, D, M, N, K, stream);
  }
}

// Units of 128 K values per wave and wave count of the LDS-staged form.
struct LdsPlan {
  int uw, nw;
};
LdsPlan lds_plan(int64_t K) {
  const int u = (int)((K + 127) / 128);
  int uw = (u + kLdsMaxWaves - 1) / kLdsMaxWaves;
  uw += uw & 1;  // units move in pairs
  return LdsPlan{uw, (u + uw - 1) / uw};
}

// The LDS-staged NVFP4 form applies for M <= 16, K <= 8192 (at most 8 waves of
// 8 units), M * K a multiple of 256 and operands whose byte offsets fit 31 bits; BSFP4_SKINNY_LDS=0
// selects the register-load single-pass form instead, BSFP4_SKINNY_SPLIT=1 the
// split-K form (measurement overrides).
// Plan of the M <= 16 LDS form: the fewest units per wave (even, <= 6) whose
// wave count fits lds_waves; {0, 0} if none does.
LdsPlan lds_plan_m16(int64_t K) {
  const int u = (int)((K + 127) / 128);
  for (int uw = 2; uw <= 6; uw += 2)
    if ((u + uw - 1) / uw <= lds_waves(uw)) return LdsPlan{uw, (u + uw - 1) / uw};
  return LdsPlan{0, 0};
}

bool use_lds(int64_t M, int64_t N, int64_t K) {
  const char* e = getenv("BSFP4_SKINNY_LDS");
  if (e && e[0] == '0') return false;
  const char* sp = getenv("BSFP4_SKINNY_SPLIT");  // measurement override: force the split-K form
  if (sp && sp[0] == '1') return false;
  if (M > 16 || K > 128 * 8 * kLdsMaxWaves || N * (K / 2) >= ((int64_t)1 << 31)) return false;
  // the activation scale block (M x K/16 bytes) is copied in whole 16-byte pieces:
  // its length must be a multiple of 16 so that no piece straddles the buffer's end
  if ((M * (K / 16)) % 16 != 0) return false;
  const LdsPlan pl = lds_plan_m16(K);
  return pl.uw > 0 && pl.nw * 1024 >= K;  // one 1 KB scale piece per wave covers the 16 x K/16 block
}

// The few-row form: M <= 4 and otherwise the LDS form's conditions (for bf16
// activations: K <= 8192 and 32-bit offsets); BSFP4_SKINNY_FEW=0 disables it.
bool use_few(int akind, int64_t M, int64_t N, int64_t K) {
  const char* e = getenv("BSFP4_SKINNY_FEW");
  if (e && e[0] == '0') return false;
  const char* sp = getenv("BSFP4_SKINNY_SPLIT");
  if (sp && sp[0] == '1') return false;
  if (M > kFewRows || K > 128 * 8 * kLdsMaxWaves || N * (K / 2) >= ((int64_t)1 << 31)) return false;
  if (akind == 0 && (M * (K / 16)) % 16 != 0) return false;  // whole 16-byte scale pieces
  return lds_plan(K).nw * 1024 >= K;
}

template <int AKIND>
hipError_t launch_few(const void* A, const uint8_t* SFA, const uint8_t* B, const uint8_t* SFB, const float* alpha,
                      uint16_t* D, int64_t M, int64_t N, int64_t K, hipStream_t stream, const float* gs = nullptr) {
  const LdsPlan pl = lds_plan(K);
  const dim3 grid((unsigned)(N / 16)), block((unsigned)(64 * pl.nw));
  switch (pl.uw) {
#define BSFP4_FEW_CASE(u)                                                                                  \
  case u:                                                                                                  \
    skinny_lds_few<AKIND, u><<<grid, block, 0, stream>>>(A, SFA, B, SFB, alpha, D, (int)M, (int)N, (int)K, gs); \
    break;
    BSFP4_FEW_CASE(2) BSFP4_FEW_CASE(4) BSFP4_FEW_CASE(6) BSFP4_FEW_CASE(8)
#undef BSFP4_FEW_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_lds(const uint8_t* A, const uint8_t* SFA, const uint8_t* B, const uint8_t* SFB,
                      const float* alpha, uint16_t* D, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  const LdsPlan pl = lds_plan_m16(K);
  const dim3 grid((unsigned)(N / 16)), block((unsigned)(64 * pl.nw));
  switch (pl.uw) {
#define BSFP4_LDS_CASE(u) \
  case u: skinny_lds<u><<<grid, block, 0, stream>>>(A, SFA, B, SFB, alpha, D, (int)M, (int)N, (int)K); break;
    BSFP4_LDS_CASE(2) BSFP4_LDS_CASE(4) BSFP4_LDS_CASE(6)
#undef BSFP4_LDS_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// The single-pass NVFP4 form applies for M <= 16 when K fits 8 waves and the
// buffer offsets fit 31 bits.
bool use_onepass(int64_t M, int64_t N, int64_t K) {
  const char* e = getenv("BSFP4_SKINNY_SPLIT");  // measurement override: force the split-K form
  if (e && e[0] == '1') return false;
  return M <= 16 && onepass_nl(K) > 0 && N * (K / 2) < ((int64_t)1 << 31);
}

// Rows 33..64 where the 64-row kernel does not apply (K % 128 != 0, or
// switched off): the split form with four M tiles for bf16 activations (the
// single-tile kernel would load them just in time); NVFP4 activations keep the
// per-wave kernel unless BSFP4_SKINNY_MT4=1.
bool split_mt4(int akind) {
  const char* e = getenv("BSFP4_SKINNY_MT4");
  if (e) return e[0] == '1';
  return akind == 1;
}

template <int AKIND>
hipError_t launch_kind(const void* A, const uint8_t* SFA, const uint8_t* B, const uint8_t* SFB,
                       const float* alpha, uint16_t* D, int64_t M, int64_t N, int64_t K, float* part,
                       hipStream_t stream) {
  if (use_few(AKIND, M, N, K)) {
    if constexpr (AKIND == 0) {
      // one or two rows: the re-blocked FP4-MFMA form (BSFP4_FEW_FP4MFMA=0
      // selects the dequantising form, for measurements and tests)
      const char* e = getenv("BSFP4_FEW_FP4MFMA");
      if (M <= 2 && !(e && e[0] == '0')) return launch_few<3>(A, SFA, B, SFB, alpha, D, M, N, K, stream);
    }
    return launch_few<AKIND>(A, SFA, B, SFB, alpha, D, M, N, K, stream);
  }
  if (AKIND == 0 && use_lds(M, N, K))
    return launch_lds(static_cast<const uint8_t*>(A), SFA, B, SFB, alpha, D, M, N, K, stream);
  if (AKIND == 0 && use_onepass(M, N, K))
    return launch_onepass(static_cast<const uint8_t*>(A), SFA, B, SFB, alpha, D, M, N, K, stream);
  const bool offsets32 = N * (K / 2) < ((int64_t)1 << 31);  // buffer offsets of the split kernels
  if (offsets32 && M <= 16) return launch_split<AKIND, 1>(A, SFA, B, SFB, alpha, D, M, N, K, part, stream);
  if (offsets32 && M <= 32) return launch_split<AKIND, 2>(A, SFA, B, SFB, alpha, D, M, N, K, part, stream);
  if (offsets32 && split_mt4(AKIND))
    return launch_split<AKIND, 4>(A, SFA, B, SFB, alpha, D, M, N, K, part, stream);
  if (M <= 16) return launch_mt<AKIND, 1>(A, SFA, B, SFB, alpha, D, M, N, K, stream);
  if (M <= 32) return launch_mt<AKIND, 2>(A, SFA, B, SFB, alpha, D, M, N, K, stream);
  return launch_mt<AKIND, 4>(A, SFA, B, SFB, alpha, D, M, N, K, stream);
}

}  // namespace

hipError_t launch_skinny_nvfp4(const uint8_t* A, const uint8_t* SFA, const uint8_t* B, const uint8_t* SFB,
                               const float* alpha, uint16_t* D, int64_t M, int64_t N, int64_t K, float* part,
                               hipStream_t stream) {
  return launch_kind<0>(A, SFA, B, SFB, alpha, D, M, N, K, part, stream);
}

hipError_t launch_skinny_w4a16(const uint16_t* A, const uint8_t* B, const uint8_t* SFB, const float* alpha,
                               uint16_t* D, int64_t M, int64_t N, int64_t K, float* part, hipStream_t stream) {
  return launch_kind<1>(A, nullptr, B, SFB, alpha, D, M, N, K, part, stream);
}

bool nvfp4_fused_quant_gemm_ok(int64_t M, int64_t N, int64_t K) {
  return M >= 1 && K % 32 == 0 && N % 16 == 0 && use_few(1, M, N, K);
}

hipError_t launch_nvfp4_fused_quant_gemm(const uint16_t* x, const float* gs, const uint8_t* B, const uint8_t* SFB,
                                         const float* alpha, uint16_t* D, int64_t M, int64_t N, int64_t K,
                                         hipStream_t stream) {
  return launch_few<2>(x, nullptr, B, SFB, alpha, D, M, N, K, stream, gs);
}

size_t skinny_workspace(int64_t M, int64_t N, int64_t K, bool fp4_activations) {
  if (M <= 0 || M > 64 || N * (K / 2) >= ((int64_t)1 << 31)) return 0;
  if (use_few(fp4_activations ? 0 : 1, M, N, K)) return 0;
  if (fp4_activations && (use_lds(M, N, K) || use_onepass(M, N, K))) return 0;
  if (M > 32 && !split_mt4(fp4_activations ? 0 : 1)) return 0;
  const SkinnyPlan pl = skinny_plan(N, K, device_cu_count(), M <= 16 ? 1 : M <= 32 ? 2 : 4);
  return pl.ksplit > 1 ? (size_t)pl.ksplit * M * N * sizeof(float) : 0;
}

}  // namespace bsfp4

// bf16 -> NVFP4 / MXFP4 block quantiser and the tensor-amax global scale.
//
// Implements the activation quantiser of the vLLM `sm103` branch comparison
// page (`nvfp4_quant_kernels.cu`, `cvt_fp16_to_fp4_sm103`; its `UE8M0_SF`
// switch gives the power-of-two MX form) and the per-expert MXFP4 activation
// quant of "[Kernel] Enable CUTLASS MXFP4 W4A4 MoE on SM12x"
// (`mxfp4_experts_quant`, here a row gather through `row_map`).  The page
// calls the per-block routine (`cvt_warp_fp16_to_fp4`) without printing it;
// the arithmetic below is the NVFP4 recipe: block scale = amax / 6 times the
// global scale, rounded to E4M3; values divided by the decoded scale and
// rounded to nearest-even onto E2M1.
//
// Each step is one correctly rounded binary32 operation (the library is built
// with -ffp-contract=off and correctly rounded division), so the output bytes
// are a deterministic function of the input: the kernel is bit-exact by
// construction, not approximately right.  The E2M1 rounding of a pair of
// values is one v_cvt_scalef32_pk_fp4_* instruction (nearest-even, saturating
// at 6, sign kept; see e2m1x2_* in quant_device.h).
//
// Mapping: one thread quantises one block (16 or 32 elements = 32 or 64
// bytes of bf16, read with 128-bit loads); consecutive lanes take consecutive
// blocks of a row, so a wave reads 2 KB (NVFP4) or 4 KB (MXFP4) of contiguous
// input and writes 512 B / 1 KB of contiguous codes plus 64 scale bytes.
// The per-expert NVFP4 form with rows of at least 64 blocks gives each wave
// whole rows instead (quantize_expert_rows), so that the expert search and the
// row lookup run once per row.
#include "device_common.h"
#include "launchers.h"
#include "quant_device.h"

#pragma clang fp contract(off)

namespace bsfp4 {
namespace {

// One block of BLK values (BLK/2 bf16 pairs in w, first value in the low
// half): its scale code and BLK/8 code words.  NVFP4 (BLK 16): E4M3 scale of
// fl32(fl32(amax / 6) * gs), codes of fl32(v * fl32(gs / sdec)).  MXFP4
// (BLK 32): E8M0 scale = smallest power of two >= fl32(amax / 6), codes of
// v / 2^(scale - 127) (exact).
template <int BLK>
__device__ __forceinline__ void quant_block(const uint32_t (&w)[BLK / 2], float gs, uint32_t& scode,
                                            uint32_t (&packed)[BLK / 8]) {
  constexpr bool kNV = (BLK == 16);
  constexpr int kWords = BLK / 2;
  float v[BLK];
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < kWords; j++) {
    v[2 * j] = bf16_bits_to_float(w[j] & 0xFFFFu);
    v[2 * j + 1] = bf16_bits_to_float(w[j] >> 16);
    amax = fmaxf(amax, fmaxf(fabsf(v[2 * j]), fabsf(v[2 * j + 1])));
  }
  if constexpr (kNV) {
    const float s = (amax / 6.0f) * gs;
    scode = e4m3_rne_satfinite(s);
    const float sdec = e4m3_decode(scode);
    const float inv = (sdec == 0.0f) ? 0.0f : gs / sdec;
#pragma unroll
    for (int j = 0; j < BLK / 8; j++) {
      uint32_t word = 0;
#pragma unroll
      for (int t = 0; t < 4; t++) word = e2m1x2_f32(word, v[8 * j + 2 * t] * inv, v[8 * j + 2 * t + 1] * inv, t);
      packed[j] = word;
    }
  } else {
    scode = e8m0_ceil(amax / 6.0f);
#pragma unroll
    for (int j = 0; j < BLK / 8; j++) {
      uint32_t word = 0;
#pragma unroll
      for (int t = 0; t < 4; t++) word = e2m1x2_bf16_pow2(word, w[4 * j + t], scode, t);
      packed[j] = word;
    }
  }
}

// The BLK/2 bf16 pairs of block b of row `row` (zeros for a row outside the input).
template <int BLK>
__device__ __forceinline__ void load_block(uint32_t (&w)[BLK / 2], const uint16_t* __restrict__ row, bool live,
                                           int64_t b) {
  if (live) {
    const uint4* p = reinterpret_cast<const uint4*>(row + b * BLK);
#pragma unroll
    for (int j = 0; j < BLK / 8; j++) {
      const uint4 t = p[j];
      w[4 * j + 0] = t.x;
      w[4 * j + 1] = t.y;
      w[4 * j + 2] = t.z;
      w[4 * j + 3] = t.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < BLK / 2; j++) w[j] = 0u;
  }
}

template <int BLK>
__device__ __forceinline__ void store_block(uint8_t* __restrict__ qrow, uint8_t* __restrict__ sfrow, int64_t b,
                                            uint32_t scode, const uint32_t (&packed)[BLK / 8]) {
  if constexpr (BLK == 16)
    *reinterpret_cast<uint2*>(qrow + b * 8) = make_uint2(packed[0], packed[1]);
  else
    *reinterpret_cast<uint4*>(qrow + b * 16) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  sfrow[b] = (uint8_t)scode;
}

// Flat form: thread i of the grid-stride loop quantises block i % (K/BLK) of
// output row i / (K/BLK).
// kExperts (NVFP4 only): output row r belongs to the expert e with
// offsets[e] <= r < offsets[e+1] and is quantised with gs_ptr[e]; rows outside
// [offsets[0], offsets[E]) are written as zeros.
template <int BLK, bool kExperts = false>
__global__ void __launch_bounds__(256)
    quantize_blocks(const uint16_t* __restrict__ x, int64_t rows_in, int64_t K,
                    const float* __restrict__ gs_ptr, const int32_t* __restrict__ row_map,
                    int64_t rows_out, uint8_t* __restrict__ q, uint8_t* __restrict__ sf,
                    const int32_t* __restrict__ offsets = nullptr, int num_experts = 0) {
  constexpr bool kNV = (BLK == 16);
  static_assert(kNV || !kExperts, "per-expert global scales are an NVFP4 form");
  const int64_t bpr = K / BLK;
  const int64_t total = rows_out * bpr;
  float gs = kNV && !kExperts ? gs_ptr[0] : 1.0f;
  // expert offsets cached in LDS for the per-row search
  __shared__ int32_t s_off[kExperts ? kMaxExperts + 1 : 1];
  if constexpr (kExperts) {
    for (int i = threadIdx.x; i <= num_experts; i += blockDim.x) s_off[i] = offsets[i];
    __syncthreads();
  }
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int64_t r = i / bpr;
    const int64_t b = i - r * bpr;
    int64_t src = row_map ? (int64_t)row_map[r] : r;
    if constexpr (kExperts) {
      // largest e with offsets[e] <= r (experts without rows share an offset
      // with the next one, so the search lands on the expert that owns r)
      int lo = 0, hi = num_experts;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_off[mid] <= r) lo = mid; else hi = mid;
      }
      if (r < s_off[0] || r >= s_off[num_experts]) src = -1;  // no expert: zero row
      gs = gs_ptr[lo];
    }
    const bool live = src >= 0 && src < rows_in;
    uint32_t w[BLK / 2];
    load_block<BLK>(w, x + (live ? src : 0) * K, live, b);
    uint32_t scode, packed[BLK / 8];
    quant_block<BLK>(w, gs, scode, packed);
    store_block<BLK>(q + r * (K / 2), sf + r * bpr, b, scode, packed);
  }
}

// Row form of the per-expert NVFP4 quantiser, for rows of at least 64
// blocks: a wave quantises whole output rows (lane l takes blocks l, l + 64,
// ...), so the row's expert (the same search over the offsets), its global
// scale and its source row are found once per row and wave-uniform, not once
// per block.  Same outputs as quantize_blocks<16, true>.
__global__ void __launch_bounds__(256)
    quantize_expert_rows(const uint16_t* __restrict__ x, int64_t rows_in, int64_t K,
                         const float* __restrict__ gs_ptr, const int32_t* __restrict__ row_map,
                         int64_t rows_out, uint8_t* __restrict__ q, uint8_t* __restrict__ sf,
                         const int32_t* __restrict__ offsets, int num_experts) {
  __shared__ int32_t s_off[kMaxExperts + 1];
  for (int i = threadIdx.x; i <= num_experts; i += blockDim.x) s_off[i] = offsets[i];
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
  const int64_t bpr = K / 16;
  const int first = __builtin_amdgcn_readfirstlane(s_off[0]);
  const int last = __builtin_amdgcn_readfirstlane(s_off[num_experts]);
  for (int64_t r = wave; r < rows_out; r += nwaves) {
    int lo = 0, hi = num_experts;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (__builtin_amdgcn_readfirstlane(s_off[mid]) <= r) lo = mid; else hi = mid;
    }
    const float gs = gs_ptr[lo];
    int64_t src = row_map ? (int64_t)row_map[r] : r;
    if (r < first || r >= last) src = -1;  // no expert: zero row
    const bool live = src >= 0 && src < rows_in;
    const uint16_t* xr = x + (live ? src : 0) * K;
    uint8_t* qr = q + r * (K / 2);
    uint8_t* sr = sf + r * bpr;
    for (int64_t b = lane; b < bpr; b += 64) {
      uint32_t w[8];
      load_block<16>(w, xr, live, b);
      uint32_t scode, packed[2];
      quant_block<16>(w, gs, scode, packed);
      store_block<16>(qr, sr, b, scode, packed);
    }
  }
}

// Per-workgroup max |x| (grid-stride, 8 bf16 per 128-bit load).
__global__ void __launch_bounds__(256)
    amax_partial(const uint16_t* __restrict__ x, int64_t numel, float* __restrict__ partial) {
  float m = 0.0f;
  const int64_t nvec = numel / 8;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  for (int64_t i = tid; i < nvec; i += stride) {
    const uint4 t = xv[i];
    const uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
    for (int j = 0; j < 4; j++) {
      m = fmaxf(m, fabsf(bf16_bits_to_float(w[j] & 0xFFFFu)));
      m = fmaxf(m, fabsf(bf16_bits_to_float(w[j] >> 16)));
    }
  }
  for (int64_t i = nvec * 8 + tid; i < numel; i += stride) m = fmaxf(m, fabsf(bf16_bits_to_float(x[i])));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  __shared__ float red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) partial[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__global__ void __launch_bounds__(256)
    global_scale_finalize(const float* __restrict__ partial, int n, float* __restrict__ gs) {
  float m = 0.0f;
  for (int i = threadIdx.x; i < n; i += blockDim.x) m = fmaxf(m, partial[i]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  __shared__ float red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    gs[0] = 2688.0f / amax;  // FLOAT8_E4M3_MAX * FLOAT4_E2M1_MAX / amax
  }
}

}  // namespace

hipError_t launch_quantize(int fmt, const uint16_t* x, int64_t rows_in, int64_t K, const float* gs,
                           const int32_t* row_map, int64_t rows_out, uint8_t* q, uint8_t* sf,
                           hipStream_t stream) {
  if (rows_out == 0) return hipSuccess;
  const int blk = (fmt == 0) ? 16 : 32;
  const int64_t items = rows_out * (K / blk);
  const int64_t want = (items + 255) / 256;
  const int grid = (int)(want < kQuantMaxGrid ? want : kQuantMaxGrid);
  if (fmt == 0) {
    quantize_blocks<16><<<grid, 256, 0, stream>>>(x, rows_in, K, gs, row_map, rows_out, q, sf);
  } else {
    quantize_blocks<32><<<grid, 256, 0, stream>>>(x, rows_in, K, nullptr, row_map, rows_out, q, sf);
  }
  return hipGetLastError();
}

hipError_t launch_nvfp4_experts_quant(const uint16_t* x, int64_t rows_in, int64_t K, const int32_t* row_map,
                                      const int32_t* offsets, int64_t E, const float* gs, int64_t rows_out,
                                      uint8_t* q, uint8_t* sf, hipStream_t stream) {
  if (rows_out == 0) return hipSuccess;
  if (K / 16 >= 64) {
    // one wave per row, four per workgroup
    const int64_t want = (rows_out + 3) / 4;
    const int grid = (int)(want < kQuantMaxGrid ? want : kQuantMaxGrid);
    quantize_expert_rows<<<grid, 256, 0, stream>>>(x, rows_in, K, gs, row_map, rows_out, q, sf, offsets, (int)E);
    return hipGetLastError();
  }
  const int64_t items = rows_out * (K / 16);
  const int64_t want = (items + 255) / 256;
  const int grid = (int)(want < kQuantMaxGrid ? want : kQuantMaxGrid);
  quantize_blocks<16, true><<<grid, 256, 0, stream>>>(x, rows_in, K, gs, row_map, rows_out, q, sf, offsets, (int)E);
  return hipGetLastError();
}

int global_scale_parts(int64_t numel) {
  const int64_t want = (numel / 8 + 255) / 256;
  return (int)(want < 1 ? 1 : (want < kAmaxMaxParts ? want : kAmaxMaxParts));
}

hipError_t launch_global_scale(const uint16_t* x, int64_t numel, float* gs, float* partial,
                               hipStream_t stream) {
  const int parts = global_scale_parts(numel);
  amax_partial<<<parts, 256, 0, stream>>>(x, numel, partial);
  global_scale_finalize<<<1, 256, 0, stream>>>(partial, parts, gs);
  return hipGetLastError();
}

}  // namespace bsfp4

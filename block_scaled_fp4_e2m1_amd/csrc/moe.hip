// MoE routing prep and the combine's fill / finalize kernels.
//
// Routing prep groups the routed (token, slot) pairs by expert, producing the
// per-expert row offsets that the pages' per-expert ops take
// (`input_offset_by_experts` of `silu_and_mul_scaled_fp4_experts_quant`, vLLM
// `sm103` branch comparison page, `csrc/ops.h`).  One workgroup per expert
// reads the whole id list (L2-resident): it counts the ids below its expert
// (its row offset), then stably compacts the flat indices equal to it with
// block-wide prefix sums.  No atomics, no workspace, deterministic output.
// The combine of the down projection sums each token's top-k FP32 rows, each
// times its routing weight, in slot order and rounds once to bf16
// (topk_sum_bf16).
#include "device_common.h"
#include "launchers.h"

namespace bsfp4 {
namespace {

constexpr int kPrepThreads = 1024;
constexpr int kPrepWaves = kPrepThreads / 64;

// Exclusive prefix of v over the workgroup (thread order) and the total.
__device__ __forceinline__ int block_excl_scan(int v, int* sh, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  if (lane == 63) sh[wave] = incl;
  __syncthreads();
  int base = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kPrepWaves; w++) {
    const int sw = sh[w];
    base += (w < wave) ? sw : 0;
    total += sw;
  }
  __syncthreads();
  return base + incl - v;
}

// One workgroup per expert e.  Pass 1 counts ids below e (the row offset of e)
// and ids equal to e; pass 2 walks the ids in rounds of 4 consecutive ids per
// thread (coalesced 128-bit loads) and writes the flat index of every id equal
// to e at offset + (matches before it), which keeps the original order.
__global__ void __launch_bounds__(kPrepThreads)
    moe_prep_kernel(const int32_t* __restrict__ ids, int n, int topk, int E, int32_t* __restrict__ offsets,
                    int32_t* __restrict__ sorted_ids, int32_t* __restrict__ sorted_tokens) {
  __shared__ int sh[kPrepWaves];
  const int e = blockIdx.x;
  const int nvec = n / 4;
  const int4* ids4 = reinterpret_cast<const int4*>(ids);
  int below = 0, mine = 0;
  for (int i = threadIdx.x; i < nvec; i += kPrepThreads) {
    const int4 v = ids4[i];
    below += (v.x < e) + (v.y < e) + (v.z < e) + (v.w < e);
    mine += (v.x == e) + (v.y == e) + (v.z == e) + (v.w == e);
  }
  for (int i = nvec * 4 + threadIdx.x; i < n; i += kPrepThreads) {
    below += ids[i] < e;
    mine += ids[i] == e;
  }
  int total_below, total_mine;
  (void)block_excl_scan(below, sh, total_below);
  (void)block_excl_scan(mine, sh, total_mine);
  if (threadIdx.x == 0) {
    offsets[e] = total_below;
    if (e == E - 1) offsets[E] = total_below + total_mine;
  }
  int base = total_below;
  const int rounds = (n + 4 * kPrepThreads - 1) / (4 * kPrepThreads);
  for (int r = 0; r < rounds; r++) {
    const int i0 = (r * kPrepThreads + threadIdx.x) * 4;  // first of this thread's 4 ids
    int v[4];
#pragma unroll
    for (int j = 0; j < 4; j++) v[j] = (i0 + j < n) ? ids[i0 + j] : -1;
    const int cnt = (v[0] == e) + (v[1] == e) + (v[2] == e) + (v[3] == e);
    int round_total;
    int pos = base + block_excl_scan(cnt, sh, round_total);
#pragma unroll
    for (int j = 0; j < 4; j++) {
      if (v[j] == e) {
        sorted_ids[pos] = i0 + j;
        if (sorted_tokens) sorted_tokens[pos] = (i0 + j) / topk;
        pos++;
      }
    }
    base += round_total;
  }
}

// out[t, n] = bf16(sum_{j < topk} w[t*topk + j] * y[t*topk + j, n]): each
// product rounded to FP32, summed in slot order.  Each thread produces 4
// consecutive columns (128-bit loads of each slot row).
__global__ void __launch_bounds__(256)
    topk_sum_bf16(const float* __restrict__ y, const float* __restrict__ w, uint16_t* __restrict__ out,
                  int64_t T, int topk, int N) {
  const int64_t quads = T * (int64_t)(N / 4);
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < quads; q += stride) {
    const int64_t t = q / (N / 4);
    const int n = (int)(q - t * (N / 4)) * 4;
    const float* src = y + (t * topk) * (int64_t)N + n;
    const float* wt = w + t * topk;
    const float4 v0 = *reinterpret_cast<const float4*>(src);
    const float w0 = wt[0];
    float4 s = make_float4(w0 * v0.x, w0 * v0.y, w0 * v0.z, w0 * v0.w);
    for (int j = 1; j < topk; j++) {
      const float4 v = *reinterpret_cast<const float4*>(src + (int64_t)j * N);
      const float wj = wt[j];
      s.x += wj * v.x;
      s.y += wj * v.y;
      s.z += wj * v.z;
      s.w += wj * v.w;
    }
    *reinterpret_cast<uint2*>(out + t * N + n) = make_uint2(pack_bf16x2(s.x, s.y), pack_bf16x2(s.z, s.w));
  }
}

}  // namespace

hipError_t launch_moe_prep(const int32_t* topk_ids, int64_t T, int64_t topk, int64_t E, int32_t* offsets,
                           int32_t* sorted_ids, int32_t* sorted_tokens, hipStream_t stream) {
  moe_prep_kernel<<<(unsigned)E, kPrepThreads, 0, stream>>>(topk_ids, (int)(T * topk), (int)topk, (int)E,
                                                             offsets, sorted_ids, sorted_tokens);
  return hipGetLastError();
}

hipError_t launch_topk_sum(const float* y, const float* w, uint16_t* out, int64_t T, int64_t topk, int64_t N,
                           hipStream_t stream) {
  const int64_t quads = T * (N / 4);
  const int64_t want = (quads + 255) / 256;
  const unsigned grid = (unsigned)(want < 1 ? 1 : (want > 16384 ? 16384 : want));
  topk_sum_bf16<<<grid, 256, 0, stream>>>(y, w, out, T, (int)topk, (int)N);
  return hipGetLastError();
}

}  // namespace bsfp4

// MoE routing prep and the combine's fill / finalize kernels.
//
// Routing prep groups the routed (token, slot) pairs by expert, producing the
// per-expert row offsets that the pages' per-expert ops take
// (`input_offset_by_experts` of `silu_and_mul_scaled_fp4_experts_quant`, vLLM
// `sm103` branch comparison page, `csrc/ops.h`).  One workgroup per expert
// reads the whole id list (L2-resident): it counts the ids below its expert
// (its row offset), then stably compacts the flat indices equal to it with
// per-wave ballots.  No atomics, no workspace, deterministic output.
// The combine of the down projection sums each token's top-k FP32 rows, each
// times its routing weight, in slot order and rounds once to bf16
// (topk_sum_bf16).
#include "device_common.h"
#include "launchers.h"

namespace bsfp4 {
namespace {

constexpr int kPrepThreads = 1024;
constexpr int kPrepWaves = kPrepThreads / 64;
constexpr int kPastEnd = 0x7FFFFFFF;  // id value for positions past a segment (matches no expert)

// One workgroup per expert e.  The ids are cut into one contiguous segment per
// wave (a multiple of 64 long); the wave reads it 64 consecutive ids at a time,
// one per lane.  Pass 1: counts of ids below e and equal to e from ballots
// (wave-uniform scalars); the per-wave counts give the expert's row offset (all
// ids below e) and each wave's first output row.  Pass 2: the wave walks its
// segment in order and writes the flat index of every id equal to e at its
// rank (ballot + lane prefix count), which keeps the original order.  No
// atomics, no block-wide barrier in the loops; segments of up to kKeep steps
// stay in registers between the passes.
__global__ void __launch_bounds__(kPrepThreads)
    moe_prep_kernel(const int32_t* __restrict__ ids, int n, int topk, int E, int32_t* __restrict__ offsets,
                    int32_t* __restrict__ sorted_ids, int32_t* __restrict__ sorted_tokens) {
  constexpr int kKeep = 32;
  __shared__ int w_below[kPrepWaves], w_mine[kPrepWaves];
  const int e = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int seg = (n + kPrepWaves * 64 - 1) / (kPrepWaves * 64) * 64;
  const int s0 = min(n, wave * seg), s1 = min(n, s0 + seg);
  const int steps = (s1 - s0 + 63) / 64;  // same for every lane of the wave
  int v[kKeep];
  auto load_chunk = [&](int k0) {
#pragma unroll
    for (int u = 0; u < kKeep; u++) {
      const int i = s0 + (k0 + u) * 64 + lane;
      v[u] = (k0 + u < steps && i < s1) ? ids[i] : kPastEnd;
    }
  };

  int below = 0, mine = 0;  // wave-uniform
  for (int k0 = 0; k0 < steps; k0 += kKeep) {
    load_chunk(k0);
#pragma unroll
    for (int u = 0; u < kKeep; u++) {
      below += __popcll(__ballot(v[u] < e));
      mine += __popcll(__ballot(v[u] == e));
    }
  }
  if (lane == 0) {
    w_below[wave] = below;
    w_mine[wave] = mine;
  }
  __syncthreads();
  int total_below = 0, total_mine = 0, base = 0;
#pragma unroll
  for (int w = 0; w < kPrepWaves; w++) {
    total_below += w_below[w];
    total_mine += w_mine[w];
    base += w < wave ? w_mine[w] : 0;
  }
  if (threadIdx.x == 0) {
    offsets[e] = total_below;
    if (e == E - 1) offsets[E] = total_below + total_mine;
  }
  if (mine == 0) return;

  // token = flat / topk without a division: for topk > 1,
  // q = umulhi(x, ceil(2^32 / topk)) is floor(x / topk) or one more for
  // x < 2^31, fixed by one compare
  const uint32_t magic = topk > 1 ? (uint32_t)((0xFFFFFFFFull + (uint64_t)topk) / (uint64_t)topk) : 0u;
  auto token_of = [&](int x) {
    if (topk == 1) return x;
    const int q = (int)__umulhi((uint32_t)x, magic);
    return q * topk > x ? q - 1 : q;
  };
  int pos = total_below + base;
  for (int k0 = 0; k0 < steps; k0 += kKeep) {
    if (steps > kKeep) load_chunk(k0);  // otherwise v still holds the only chunk
#pragma unroll
    for (int u = 0; u < kKeep; u++) {
      const uint64_t bal = __ballot(v[u] == e);
      if (bal == 0) continue;
      if (v[u] == e) {
        const int r = pos + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
        const int x = s0 + (k0 + u) * 64 + lane;
        sorted_ids[r] = x;
        if (sorted_tokens) sorted_tokens[r] = token_of(x);
      }
      pos += __popcll(bal);
    }
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

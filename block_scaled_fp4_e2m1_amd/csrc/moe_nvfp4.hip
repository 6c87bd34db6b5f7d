// NVFP4 x NVFP4 grouped GEMM over per-expert weights (the NVFP4 form of the
// mixture-of-experts layer: `scaled_fp4_experts_quant` and
// `silu_and_mul_scaled_fp4_experts_quant` on the vLLM `sm103` branch comparison
// page, whose per-expert offsets address the rows).  Rows [off[e], off[e+1])
// of A times W[e]^T, FP32 accumulation, alpha[e] on the accumulator.  The K
// loop is the dense kernel's: fp4 loads one group ahead, dequantised once to
// fp16 in LDS, v_mfma_f32_32x32x16_f16.  The grid is persistent and walks the
// (expert, column tile, row tile) list built in LDS from the offsets, row
// tiles innermost, consecutive items on one XCD (a weight panel is shared by
// an expert's row tiles).
#include "device_common.h"
#include "launchers.h"
#include "nvfp4_f16core.h"
#include "quant_device.h"

namespace bsfp4 {
namespace {

struct GroupedArgs {
  const uint8_t* A;        // [rows, K/2] codes, rows in expert order
  const uint8_t* SFA;      // [rows, K/16] E4M3 scales
  const int32_t* offsets;  // [E+1]
  int E, rows;
  const uint8_t* W;        // [E, N, K/2]
  const uint8_t* WSF;      // [E, N, K/16]
  const float* alpha;      // [E] or nullptr (1.0)
  int N, K;
  uint16_t* out;           // STORE: bf16 [rows, N]
  uint8_t* out_q;          // SILU: [rows, N/4] codes of act
  uint8_t* out_sf;         // SILU: [rows, N/32] E4M3 scales of act
  const float* out_gs;     // SILU: [E] global scale of act
  const int32_t* sorted_ids;  // COMBINE: flat (token, slot) index of each row
  float* y;                // COMBINE: FP32 [rows, N] indexed by flat index
};

constexpr int kGroupedMaxE = 1024;

// One load group (2 stages) of the tile's A rows and B rows.  SILU: B rows
// [0, BN/2) are gate rows n0g.. of W[e], rows [BN/2, BN) the up rows
// N/2 + n0g..; `nb` is the number of valid gate (or plain) rows.
template <int BM, int BN, int NT, bool kSilu>
__device__ __forceinline__ void grouped_group_load(Fp4Group<BM, BN, NT>& g, __amdgpu_buffer_rsrc_t ra_q,
                                                   __amdgpu_buffer_rsrc_t ra_s, __amdgpu_buffer_rsrc_t rb_q,
                                                   __amdgpu_buffer_rsrc_t rb_s, int r0, int m, int ma, int nb,
                                                   int up_jump, int K, int k0) {
  constexpr int kA = BM * 4 / NT;
#pragma unroll
  for (int i = 0; i < Fp4Group<BM, BN, NT>::kChunks; i++) {
    const bool is_a = i < kA;
    const int r = r0 + (is_a ? i : i - kA) * (NT / 4);
    const int c = (i & 1) ? (m ^ 2) : m;
    int rl = r, ro = r;  // row for the bounds check, row for the offset
    if (kSilu && !is_a && r >= BN / 2) {
      rl = r - BN / 2;
      ro = r + up_jump;
    }
    const bool live = rl < (is_a ? ma : nb) && k0 + c * 32 < K;
    const uint32_t oc = live ? (uint32_t)(ro * (K / 2) + c * 16 + k0 / 2) : kOOB;
    const uint32_t os = live ? (uint32_t)(ro * (K / 16) + c * 2 + k0 / 16) : kOOB;
    g.code[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(is_a ? ra_q : rb_q, (int)oc, 0, 0));
    g.sc[i] = __builtin_amdgcn_raw_buffer_load_b16(is_a ? ra_s : rb_s, (int)os, 0, 0);
  }
}

__device__ __forceinline__ int64_t clamp_bytes(int64_t b) { return b < 0x7FFFFFFF ? b : 0x7FFFFFFF; }

// Requires K % 32 == 0, N % 32 == 0 (N % 64 == 0 for SILU), N*K/2 < 2^31,
// E <= kGroupedMaxE.
template <int BM, int BN, int WGM, int WGN, int EPI>
__global__ void __launch_bounds__(64 * WGM * WGN, 2) nvfp4_grouped(GroupedArgs p) {
  constexpr int NT = 64 * WGM * WGN;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int kStage = f16_row<NT>(BM + BN);
  constexpr bool kSilu = EPI == kEpiSilu;
  static_assert(2 * kStage <= 80 * 1024, "two workgroups per CU");
  static_assert(!kSilu || (BN == 128 && BM * 2 == NT), "SILU epilogue mapping: 2 threads per row, 64 act columns");
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStage];
  __shared__ int tile_start[kGroupedMaxE + 1];
  __shared__ int wave_sum[NT / 64];
  __shared__ int row_f[EPI == kEpiCombine ? BM : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int g = lane >> 5, lr = lane & 31;
  const int K = p.K, N = p.N;
  // column tiles: BN output columns, or BN/2 act columns (gate/up pairs)
  const int ncols = kSilu ? N / 2 : N;
  constexpr int kTileCols = kSilu ? BN / 2 : BN;
  const int ntn = (ncols + kTileCols - 1) / kTileCols;

  // ---- work list: tile_start[e] = items of experts before e (block scan)
  {
    int cnt[4];
    int local = 0;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int e = tid * 4 + j;
      int c = 0;
      if (e < p.E) c = max((p.offsets[e + 1] - p.offsets[e] + BM - 1) / BM, 0) * ntn;
      cnt[j] = c;
      local += c;
    }
    int incl = local;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    if (lane == 63) wave_sum[wave] = incl;
    __syncthreads();
    int base = incl - local;
    for (int w = 0; w < wave; w++) base += wave_sum[w];
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int e = tid * 4 + j;
      if (e < p.E) tile_start[e] = base;
      base += cnt[j];
    }
    if (tid == NT - 1) tile_start[p.E] = base;
    __syncthreads();
  }
  const int total = tile_start[p.E];
  const int G = gridDim.x;
  const int slot = (G % 8 == 0) ? (int)(blockIdx.x % 8) * (G / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;
  const uint8_t* fra = smem + lr * kF16Pitch + g * 16;

  for (int t = slot; t < total; t += G) {
    int lo = 0, hi = p.E - 1;  // largest e with tile_start[e] <= t
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tile_start[mid] <= t) lo = mid; else hi = mid - 1;
    }
    const int e = lo;
    const int row0 = p.offsets[e], row_end = min(p.offsets[e + 1], p.rows);
    const int nmt = (p.offsets[e + 1] - row0 + BM - 1) / BM;
    const int local = t - tile_start[e];
    const int tn = local / nmt, tmi = local % nmt;
    const int m0 = row0 + tmi * BM;
    const int ma = row0 >= 0 ? row_end - m0 : 0;      // valid A rows of the tile
    const int c0 = tn * kTileCols;                    // first output (or act) column
    const int nb = min(kTileCols, ncols - c0);        // valid columns of the tile
    const float alpha = p.alpha ? p.alpha[e] : 1.0f;

    v16f acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
      for (int j = 0; j < TN; j++) acc[i][j] = v16f{};

    {
      const int64_t kb = K / 2, ks = K / 16;
      const uint8_t* wq = p.W + (int64_t)e * N * kb;
      const uint8_t* ws = p.WSF + (int64_t)e * N * ks;
      const __amdgpu_buffer_rsrc_t ra_q = make_rsrc(p.A + (int64_t)m0 * kb, clamp_bytes((int64_t)max(ma, 0) * kb));
      const __amdgpu_buffer_rsrc_t ra_s = make_rsrc(p.SFA + (int64_t)m0 * ks, clamp_bytes((int64_t)max(ma, 0) * ks));
      const __amdgpu_buffer_rsrc_t rb_q = make_rsrc(wq + (int64_t)c0 * kb, (int64_t)(N - c0) * kb);
      const __amdgpu_buffer_rsrc_t rb_s = make_rsrc(ws + (int64_t)c0 * ks, (int64_t)(N - c0) * ks);
      const int up_jump = N / 2 - BN / 2;
      const int r0 = tid >> 2, mq = tid & 3;
      const int nst = (K + kF16StageK - 1) / kF16StageK;
      const int ngroups = (nst + 1) / 2;

      Fp4Group<BM, BN, NT> cur;
      grouped_group_load<BM, BN, NT, kSilu>(cur, ra_q, ra_s, rb_q, rb_s, r0, mq, ma, nb, up_jump, K, 0);
      {
        constexpr int kWords = 4 * Fp4Group<BM, BN, NT>::kChunks / 2;
#pragma unroll
        for (int w = 0; w < kWords; w++) {
          switch (w) {
#define BSFP4_W(x) \
  case x:          \
    if constexpr (x < kWords) group_word_store<x, 0, BM, BN, NT>(cur, smem, tid); \
    break;
            BSFP4_W(0) BSFP4_W(1) BSFP4_W(2) BSFP4_W(3) BSFP4_W(4) BSFP4_W(5) BSFP4_W(6) BSFP4_W(7)
            BSFP4_W(8) BSFP4_W(9) BSFP4_W(10) BSFP4_W(11) BSFP4_W(12) BSFP4_W(13) BSFP4_W(14) BSFP4_W(15)
#undef BSFP4_W
          }
        }
      }
      __syncthreads();
      for (int gi = 0; gi < ngroups; gi++) {
        Fp4Group<BM, BN, NT> nxt;
        grouped_group_load<BM, BN, NT, kSilu>(nxt, ra_q, ra_s, rb_q, rb_s, r0, mq, ma, nb, up_jump, K,
                                              (gi + 1) * kGroupK);
        __builtin_amdgcn_sched_barrier(0);
        f16_stage_compute<BM, BN, WGM, WGN>(fra, fra, acc, cur, smem + kStage, tid, true, wm, wn);
        __syncthreads();
        f16_stage_compute<BM, BN, WGM, WGN>(fra + kStage, fra + kStage, acc, nxt, smem, tid, false, wm, wn);
        __syncthreads();
        cur = nxt;
      }
    }

    // ---- epilogues.  Lane: tile row wm*WM + 32i + lr, registers 4q..4q+3 of
    // fragment j: tile columns wn*WN + 32j + 8q + 4g .. +3.
    if constexpr (EPI == kEpiCombine) {
      if (tid < BM) {
        const int f = tid < ma ? p.sorted_ids[m0 + tid] : -1;
        row_f[tid] = f < p.rows ? f : -1;  // rows == T * topk flat indices
      }
      // FP32 rows alpha * acc through LDS in row bands, 16 bytes per lane per store
      constexpr int kPitch = BN * 4 + 16;
      constexpr int kPasses = (BM * kPitch + 2 * kStage - 1) / (2 * kStage);
      constexpr int kBandRows = BM / kPasses;
      static_assert(kBandRows % 32 == 0 && kBandRows * kPitch <= 2 * kStage, "band fits in LDS");
#pragma unroll
      for (int h = 0; h < kPasses; h++) {
        if (h > 0) __syncthreads();
#pragma unroll
        for (int i = 0; i < TM; i++) {
          const int r = wm * WM + i * 32;
          if (r / kBandRows != h) continue;
          const int rl = r - h * kBandRows + lr;
#pragma unroll
          for (int j = 0; j < TN; j++)
#pragma unroll
            for (int q = 0; q < 4; q++) {
              const int c = wn * WN + j * 32 + 8 * q + 4 * g;
              *reinterpret_cast<float4*>(smem + rl * kPitch + c * 4) =
                  make_float4(alpha * acc[i][j][4 * q], alpha * acc[i][j][4 * q + 1], alpha * acc[i][j][4 * q + 2],
                              alpha * acc[i][j][4 * q + 3]);
            }
        }
        __syncthreads();
        constexpr int kChunksPerRow = BN / 4;
        for (int idx = tid; idx < kBandRows * kChunksPerRow; idx += NT) {
          const int rl = idx / kChunksPerRow, c = (idx % kChunksPerRow) * 4;
          const int f = row_f[h * kBandRows + rl];
          if (f >= 0 && c < nb)
            *reinterpret_cast<float4*>(p.y + (int64_t)f * N + c0 + c) =
                *reinterpret_cast<const float4*>(smem + rl * kPitch + c * 4);
        }
      }
    } else {
      // h = bf16(alpha * acc) tile in LDS (row pitch BN*2 + 16 bytes)
      constexpr int kPitch = BN * 2 + 16;
      static_assert(BM * kPitch <= 2 * kStage, "bf16 tile fits in the stage buffers");
#pragma unroll
      for (int i = 0; i < TM; i++) {
        const int r = wm * WM + i * 32 + lr;
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
          for (int q = 0; q < 4; q++) {
            const int c = wn * WN + j * 32 + 8 * q + 4 * g;
            *reinterpret_cast<uint2*>(smem + r * kPitch + c * 2) =
                make_uint2(pack_bf16x2(alpha * acc[i][j][4 * q], alpha * acc[i][j][4 * q + 1]),
                           pack_bf16x2(alpha * acc[i][j][4 * q + 2], alpha * acc[i][j][4 * q + 3]));
          }
      }
      __syncthreads();
      if constexpr (EPI == kEpiStore) {
        constexpr int kChunksPerRow = BN / 8;
        for (int idx = tid; idx < BM * kChunksPerRow; idx += NT) {
          const int r = idx / kChunksPerRow, c = (idx % kChunksPerRow) * 8;
          if (r < ma && c < nb)
            *reinterpret_cast<uint4*>(p.out + (int64_t)(m0 + r) * N + c0 + c) =
                *reinterpret_cast<const uint4*>(smem + r * kPitch + c * 2);
        }
      } else {
        // SILU: thread -> tile row tid/2, act columns 32*(tid&1) .. +31 (two
        // NVFP4 blocks); gate at tile column c, up at BN/2 + c.
        // act = bf16(silu(h_g) * h_u), SiLU with the hardware exp2 and
        // reciprocal; then the dense quantiser's NVFP4 recipe with gs[e]:
        // s = fl32(fl32(amax/6) * gs) -> E4M3 (RNE, saturating), inv =
        // fl32(gs / dec(s)), codes = E2M1 RNE of fl32(a * inv).
        const int r = tid >> 1, hh = tid & 1;
        if (r < ma && 32 * hh < nb) {
          const float gsv = p.out_gs[e];
          constexpr float kLog2e = 1.4426950408889634f;
          const uint8_t* rowp = smem + r * kPitch;
          uint32_t words[4];
          uint32_t scodes = 0;
#pragma unroll
          for (int b = 0; b < 2; b++) {
            const int cb = 32 * hh + 16 * b;  // first act column of the block
            uint4 gv[2], uv[2];
            gv[0] = *reinterpret_cast<const uint4*>(rowp + cb * 2);
            gv[1] = *reinterpret_cast<const uint4*>(rowp + cb * 2 + 16);
            uv[0] = *reinterpret_cast<const uint4*>(rowp + (BN / 2 + cb) * 2);
            uv[1] = *reinterpret_cast<const uint4*>(rowp + (BN / 2 + cb) * 2 + 16);
            const uint32_t gw[8] = {gv[0].x, gv[0].y, gv[0].z, gv[0].w, gv[1].x, gv[1].y, gv[1].z, gv[1].w};
            const uint32_t uw[8] = {uv[0].x, uv[0].y, uv[0].z, uv[0].w, uv[1].x, uv[1].y, uv[1].z, uv[1].w};
            float a[16];
            float amax = 0.0f;
#pragma unroll
            for (int k = 0; k < 16; k++) {
              const uint32_t gb = (k & 1) ? (gw[k >> 1] >> 16) : (gw[k >> 1] & 0xFFFFu);
              const uint32_t ub = (k & 1) ? (uw[k >> 1] >> 16) : (uw[k >> 1] & 0xFFFFu);
              const float hg = bf16_bits_to_float(gb), hu = bf16_bits_to_float(ub);
              const float ex = __builtin_amdgcn_exp2f(-hg * kLog2e);
              a[k] = (float)(__bf16)(hg * __builtin_amdgcn_rcpf(1.0f + ex) * hu);
              amax = fmaxf(amax, fabsf(a[k]));
            }
            const float s = (amax / 6.0f) * gsv;
            const uint32_t sc = e4m3_rne_satfinite(s);
            const float sdec = e4m3_decode(sc);
            const float inv = (sdec == 0.0f) ? 0.0f : gsv / sdec;
#pragma unroll
            for (int wd = 0; wd < 2; wd++) {
              uint32_t word = 0;
#pragma unroll
              for (int u = 0; u < 4; u++)
                word = e2m1x2_f32(word, a[8 * wd + 2 * u] * inv, a[8 * wd + 2 * u + 1] * inv, u);
              words[2 * b + wd] = word;
            }
            scodes |= sc << (8 * b);
          }
          const int64_t m = m0 + r;
          const int ca = c0 + 32 * hh;  // first act column of the thread
          *reinterpret_cast<uint4*>(p.out_q + m * (N / 4) + ca / 2) = make_uint4(words[0], words[1], words[2], words[3]);
          *reinterpret_cast<uint16_t*>(p.out_sf + m * (N / 32) + ca / 16) = (uint16_t)scodes;
        }
      }
    }
    __syncthreads();  // the next item's first stage reuses the LDS
  }
}

}  // namespace

// Grouped NVFP4 GEMM: persistent grid of two workgroups per CU (fewer when
// the list is short; the list length is bounded by sum_e ceil(rows_e/BM) <=
// rows/BM + E row tiles per column tile).
hipError_t launch_nvfp4_grouped(const uint8_t* Aq, const uint8_t* Asf, const int32_t* offsets, int64_t E,
                                int64_t rows, const uint8_t* W, const uint8_t* Wsf, const float* alpha,
                                int64_t N, int64_t K, int epilogue, uint16_t* out, uint8_t* out_q, uint8_t* out_sf,
                                const float* out_gs, const int32_t* sorted_ids, float* y, hipStream_t stream) {
  constexpr int BM = 128, BN = 128;
  GroupedArgs a;
  a.A = Aq;
  a.SFA = Asf;
  a.offsets = offsets;
  a.E = (int)E;
  a.rows = (int)rows;
  a.W = W;
  a.WSF = Wsf;
  a.alpha = alpha;
  a.N = (int)N;
  a.K = (int)K;
  a.out = out;
  a.out_q = out_q;
  a.out_sf = out_sf;
  a.out_gs = out_gs;
  a.sorted_ids = sorted_ids;
  a.y = y;
  const int64_t cols = epilogue == kEpiSilu ? N / 2 : N;
  const int64_t tile_cols = epilogue == kEpiSilu ? BN / 2 : BN;
  const int64_t max_items = ((rows + BM - 1) / BM + E) * ((cols + tile_cols - 1) / tile_cols);
  int64_t grid = 2 * (int64_t)device_cu_count();
  if (max_items < grid) grid = max_items;
  if (grid > 8) grid -= grid % 8;
  if (grid < 1) grid = 1;
  if (epilogue == kEpiSilu)
    nvfp4_grouped<BM, BN, 2, 2, kEpiSilu><<<(unsigned)grid, 256, 0, stream>>>(a);
  else if (epilogue == kEpiCombine)
    nvfp4_grouped<BM, BN, 2, 2, kEpiCombine><<<(unsigned)grid, 256, 0, stream>>>(a);
  else
    nvfp4_grouped<BM, BN, 2, 2, kEpiStore><<<(unsigned)grid, 256, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace bsfp4

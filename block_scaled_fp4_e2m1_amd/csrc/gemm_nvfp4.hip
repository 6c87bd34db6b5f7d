// NVFP4 W4A4 GEMM for gfx950:  D = bf16(alpha * dec(A) @ dec(B)^T).
//
// The operation of `Fp4GemmSm103` / `cutlass_scaled_fp4_mm` (vLLM `sm103`
// branch comparison page, `nvfp4_scaled_mm_kernels.cu`) and CuTe-DSL `mm_fp4`
// ("perf(gemm): optimize SM103 CuTe DSL mm_fp4 kernel"): E2M1 operands with one
// E4M3 scale per 16 K-elements, FP32 accumulation, alpha applied to the FP32
// accumulator followed by one conversion to bf16 ("Alpha epilogue bug").
//
// Why fp16 MFMA: gfx950's scaled FP4 MFMA applies one power-of-two (E8M0) scale
// per 32 K-elements, while NVFP4 carries a 3-mantissa-bit E4M3 scale per 16.
// The product of an E2M1 value and an E4M3 scale has at most 6 significant bits
// and lies in [2^-10, 2688], so it is exact in fp16; the fp16 MFMA multiplies
// exactly and accumulates in FP32.  Dequantisation is two VALU instructions per
// pair of values: v_cvt_scalef32_pk_f16_fp4 (scale 1.0) and a packed fp16
// multiply by the block scale.
//
// Kernels, by M:
//   * 24..128 rows with K % 128 == 0: the row kernel of gemm_w4a16.hip with
//     its NVFP4 activation form;
//   * other shapes of up to 64 rows: the weight-streaming kernels of
//     gemm_skinny.hip;
//   * the rest: nvfp4_gemm_f16lds, the dequantise-once kernel on the shared
//     core of nvfp4_f16core.h (256x256 tiles of 16 waves, or 256x128 / 128x128
//     tiles of 4 waves; every E2M1 value dequantised once per workgroup into
//     fp16 LDS stages), with the tile shape and a K split planned from
//     measured per-workgroup rates (plan_tiled) and split partials summed by
//     splitk_reduce;
//   * operands of 2^31 bytes or more: nvfp4_gemm_tiled, the register-dequant
//     kernel below (64-bit addressing).  Its structure: a BM x BN tile, K in
//     stages of 128 elements (64 code bytes and 8 scale bytes per row); each
//     stage's packed codes and scale bytes are loaded with 128-bit loads into
//     registers one stage ahead, then stored to LDS (double buffered) in a
//     chunk-swizzled layout that keeps the fragment reads free of bank
//     conflicts; every wave reads its fragments from LDS as packed FP4 (4x less
//     LDS traffic than fp16 tiles), dequantises them in registers and issues
//     v_mfma_f32_32x32x16_f16 on its wave tile.
// Epilogues: alpha * acc, RNE to bf16, bounds-checked stores.
//
// MFMA lane layouts (measured on gfx950): for 32x32x16, lane l supplies row
// l%32 and eight consecutive K values of group l/32 of each operand; output
// register r of lane l holds row 8*(r/4) + 4*(l/32) + r%4, column l%32.  Within
// a stage the K index assigned to a lane's values is a fixed permutation shared
// by A and B, which leaves the sum unchanged; each lane's eight values always
// lie inside one 16-element scale block.
#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <cstring>

#include "device_common.h"
#include "launchers.h"
#include "nvfp4_f16core.h"

namespace bsfp4 {
namespace {

constexpr int kStageK = 128;              // K elements per stage
constexpr int kStageBytes = kStageK / 2;  // 64 code bytes per row per stage
constexpr int kStageBlocks = kStageK / 16;  // 8 E4M3 scales per row per stage

// Position of 16-byte chunk c (0..3) of row r inside the row's 64 bytes.  With
// this swizzle, 8 (or 16) lanes reading the same logical chunk of 8 (or 16)
// consecutive rows touch 8 (or 16) distinct 16-byte bank groups.
__device__ __forceinline__ int swz(int r, int c) { return c ^ (((r >> 1) ^ (r >> 3)) & 3); }

template <int ROWS, int NT>
struct StageRegs {
  static constexpr int kChunks = ROWS * 4 / NT;  // 16-byte code chunks per thread
  uint4 code[kChunks];
  uint32_t sc[2];  // 8 scale bytes of row `tid` (threads < ROWS)
};

template <int ROWS, int NT>
__device__ __forceinline__ void load_stage(StageRegs<ROWS, NT>& st, const uint8_t* __restrict__ q,
                                           const uint8_t* __restrict__ sf, int row0, int nrows,
                                           int64_t K, int k0, int tid) {
  const int64_t row_bytes = K / 2;
  const int64_t row_blocks = K / 16;
#pragma unroll
  for (int i = 0; i < StageRegs<ROWS, NT>::kChunks; i++) {
    const int idx = tid + i * NT;
    const int r = idx >> 2, c = idx & 3;
    const int64_t kb = (int64_t)k0 / 2 + c * 16;  // byte offset in the row
    if (row0 + r < nrows && kb < row_bytes) {
      st.code[i] = *reinterpret_cast<const uint4*>(q + (int64_t)(row0 + r) * row_bytes + kb);
    } else {
      st.code[i] = make_uint4(0, 0, 0, 0);
    }
  }
  if (tid < ROWS) {
    const int r = tid;
    uint32_t w[4] = {0, 0, 0, 0};
    if (row0 + r < nrows) {
      // K % 32 == 0, so scale bytes come in valid pairs (2-byte aligned)
      const uint16_t* p = reinterpret_cast<const uint16_t*>(sf + (int64_t)(row0 + r) * row_blocks);
      const int64_t b0 = k0 / 16;
#pragma unroll
      for (int j = 0; j < 4; j++)
        if (b0 + 2 * j < row_blocks) w[j] = p[b0 / 2 + j];
    }
    st.sc[0] = w[0] | (w[1] << 16);
    st.sc[1] = w[2] | (w[3] << 16);
  }
}

template <int ROWS, int NT>
__device__ __forceinline__ void store_stage(const StageRegs<ROWS, NT>& st, uint8_t* lds_q, uint8_t* lds_s,
                                            int tid) {
#pragma unroll
  for (int i = 0; i < StageRegs<ROWS, NT>::kChunks; i++) {
    const int idx = tid + i * NT;
    const int r = idx >> 2, c = idx & 3;
    *reinterpret_cast<uint4*>(lds_q + r * kStageBytes + swz(r, c) * 16) = st.code[i];
  }
  if (tid < ROWS) *reinterpret_cast<uint2*>(lds_s + tid * kStageBlocks) = make_uint2(st.sc[0], st.sc[1]);
}

// splits == 1: D = bf16(alpha * acc).  splits > 1: workgroup (tile, s) sums
// the s-th contiguous range of K stages and writes its FP32 partial tile to
// part[s][M][N]; a second kernel adds the partials in split order.
template <int BM, int BN, int WGM, int WGN>
__global__ void __launch_bounds__(64 * WGM * WGN, 1)
    nvfp4_gemm_tiled(const uint8_t* __restrict__ A, const uint8_t* __restrict__ SFA,
                     const uint8_t* __restrict__ B, const uint8_t* __restrict__ SFB,
                     const float* __restrict__ alpha_ptr, uint16_t* __restrict__ D, int M, int N,
                     int64_t K, int tiles_n, int splits, float* __restrict__ part) {
  constexpr int NT = 64 * WGM * WGN;          // threads
  constexpr int WM = BM / WGM, WN = BN / WGN;  // wave tile
  constexpr int TM = WM / 32, TN = WN / 32;   // 32x32 MFMA tiles per wave
  constexpr int kABytes = BM * kStageBytes, kBBytes = BN * kStageBytes;
  constexpr int kStage = kABytes + kBBytes + (BM + BN) * kStageBlocks;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int split = blockIdx.x % splits;
  const int tile = blockIdx.x / splits;
  const int tile_m = tile / tiles_n, tile_n = tile % tiles_n;
  const int m0 = tile_m * BM, n0 = tile_n * BN;

  v16f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; i++)
#pragma unroll
    for (int j = 0; j < TN; j++) acc[i][j] = v16f{};

  const int total_stages = (int)((K + kStageK - 1) / kStageK);
  const int s_begin = (int)((int64_t)total_stages * split / splits);
  const int s_end = (int)((int64_t)total_stages * (split + 1) / splits);
  const int nstages = s_end - s_begin;
  const int kbase = s_begin * kStageK;
  StageRegs<BM, NT> ra;
  StageRegs<BN, NT> rb;
  load_stage<BM, NT>(ra, A, SFA, m0, M, K, kbase, tid);
  load_stage<BN, NT>(rb, B, SFB, n0, N, K, kbase, tid);
  {
    uint8_t* s = smem;
    store_stage<BM, NT>(ra, s, s + kABytes + kBBytes, tid);
    store_stage<BN, NT>(rb, s + kABytes, s + kABytes + kBBytes + BM * kStageBlocks, tid);
  }
  __syncthreads();

  const int g = lane >> 5;     // K group of this lane inside an MFMA
  const int lr = lane & 31;    // row inside a 32-row MFMA tile

  for (int s = 0; s < nstages; s++) {
    const bool more = (s + 1) < nstages;
    if (more) {
      load_stage<BM, NT>(ra, A, SFA, m0, M, K, kbase + (s + 1) * kStageK, tid);
      load_stage<BN, NT>(rb, B, SFB, n0, N, K, kbase + (s + 1) * kStageK, tid);
    }
    const uint8_t* st = smem + (s & 1) * kStage;
    const uint8_t* sq_a = st;
    const uint8_t* sq_b = st + kABytes;
    const uint8_t* ss_a = st + kABytes + kBBytes;
    const uint8_t* ss_b = ss_a + BM * kStageBlocks;
#pragma unroll
    for (int j = 0; j < 2; j++) {
      // lane covers chunk 2j+g of its row: K elements 64j + 32g + [0, 32)
      uint4 ca[TM], cb[TN];
      v2h sa[TM], sb[TN];
#pragma unroll
      for (int i = 0; i < TM; i++) {
        const int r = wm * WM + i * 32 + lr;
        ca[i] = *reinterpret_cast<const uint4*>(sq_a + r * kStageBytes + swz(r, 2 * j + g) * 16);
        sa[i] = e4m3x2_to_f16x2(*reinterpret_cast<const uint16_t*>(ss_a + r * kStageBlocks + 4 * j + 2 * g));
      }
#pragma unroll
      for (int i = 0; i < TN; i++) {
        const int r = wn * WN + i * 32 + lr;
        cb[i] = *reinterpret_cast<const uint4*>(sq_b + r * kStageBytes + swz(r, 2 * j + g) * 16);
        sb[i] = e4m3x2_to_f16x2(*reinterpret_cast<const uint16_t*>(ss_b + r * kStageBlocks + 4 * j + 2 * g));
      }
#pragma unroll
      for (int w = 0; w < 4; w++) {
        v8h fa[TM], fb[TN];
#pragma unroll
        for (int i = 0; i < TM; i++) {
          const uint32_t word = w == 0 ? ca[i].x : w == 1 ? ca[i].y : w == 2 ? ca[i].z : ca[i].w;
          fa[i] = dequant8(word, (w < 2) ? sa[i].x : sa[i].y);
        }
#pragma unroll
        for (int i = 0; i < TN; i++) {
          const uint32_t word = w == 0 ? cb[i].x : w == 1 ? cb[i].y : w == 2 ? cb[i].z : cb[i].w;
          fb[i] = dequant8(word, (w < 2) ? sb[i].x : sb[i].y);
        }
#pragma unroll
        for (int i = 0; i < TM; i++)
#pragma unroll
          for (int jn = 0; jn < TN; jn++)
            acc[i][jn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i], fb[jn], acc[i][jn], 0, 0, 0);
      }
    }
    if (more) {
      uint8_t* nx = smem + ((s + 1) & 1) * kStage;
      store_stage<BM, NT>(ra, nx, nx + kABytes + kBBytes, tid);
      store_stage<BN, NT>(rb, nx + kABytes, nx + kABytes + kBBytes + BM * kStageBlocks, tid);
    }
    __syncthreads();
  }

  if (splits == 1) {
    const float alpha = alpha_ptr ? alpha_ptr[0] : 1.0f;
#pragma unroll
    for (int i = 0; i < TM; i++) {
#pragma unroll
      for (int jn = 0; jn < TN; jn++) {
        const int n = n0 + wn * WN + jn * 32 + lr;
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const int m = m0 + wm * WM + i * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          if (m < M && n < N) D[(int64_t)m * N + n] = (uint16_t)float_to_bf16_rne(alpha * acc[i][jn][r]);
        }
      }
    }
  } else {
    float* dst = part + (int64_t)split * M * N;
#pragma unroll
    for (int i = 0; i < TM; i++) {
#pragma unroll
      for (int jn = 0; jn < TN; jn++) {
        const int n = n0 + wn * WN + jn * 32 + lr;
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const int m = m0 + wm * WM + i * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          if (m < M && n < N) dst[(int64_t)m * N + n] = acc[i][jn][r];
        }
      }
    }
  }
}

// Dequantise-once kernel on the shared core of nvfp4_f16core.h (its design
// notes are there).
// Requires M*K/2 and N*K/2 < 2^31 (buffer offsets), K % 32 == 0, N % 4 == 0.
template <int BM, int BN, int WGM, int WGN>
__global__ void __launch_bounds__(64 * WGM * WGN, 1)
    nvfp4_gemm_f16lds(const uint8_t* __restrict__ A, const uint8_t* __restrict__ SFA,
                      const uint8_t* __restrict__ B, const uint8_t* __restrict__ SFB,
                      const float* __restrict__ alpha_ptr, uint16_t* __restrict__ D, int M, int N,
                      int64_t K, int tiles_m, int tiles_n, int splits, float* __restrict__ part) {
  constexpr int NT = 64 * WGM * WGN;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int kStage = f16_row<NT>(BM + BN);  // fp16 stage bytes (A rows then B rows)
  static_assert(2 * kStage <= 160 * 1024, "two stages must fit in LDS");
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int g = lane >> 5, lr = lane & 31;

  // work item -> (tile, split).  Workgroups are dispatched round-robin over the
  // 8 XCDs; consecutive items go to one XCD, and items are ordered in bands of 4
  // tile rows so an XCD's items share few A and B panels in its L2.
  const int items = tiles_m * tiles_n * splits;
  int item = blockIdx.x;
  if (items % 8 == 0) item = (int)(blockIdx.x % 8) * (items / 8) + (int)(blockIdx.x / 8);
  const int split = item % splits;
  const int tile = item / splits;
  constexpr int kBand = 4;
  const int band_tiles = kBand * tiles_n;
  const int band = tile / band_tiles, in_band = tile % band_tiles;
  const int band_rows = min(kBand, tiles_m - band * kBand);
  const int tile_m = band * kBand + in_band % band_rows;
  const int tile_n = in_band / band_rows;
  const int m0 = tile_m * BM, n0 = tile_n * BN;

  v16f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; i++)
#pragma unroll
    for (int j = 0; j < TN; j++) acc[i][j] = v16f{};

  const int total = (int)((K + kF16StageK - 1) / kF16StageK);
  const int sb = (int)((int64_t)total * split / splits);
  const int nst = (int)((int64_t)total * (split + 1) / splits) - sb;

  if (nst > 0) {
    // buffers start at the tile's first row; the range check uses what is left
    const __amdgpu_buffer_rsrc_t ra_q = make_rsrc(A + (int64_t)m0 * (K / 2), (int64_t)(M - m0) * (K / 2));
    const __amdgpu_buffer_rsrc_t ra_s = make_rsrc(SFA + (int64_t)m0 * (K / 16), (int64_t)(M - m0) * (K / 16));
    const __amdgpu_buffer_rsrc_t rb_q = make_rsrc(B + (int64_t)n0 * (K / 2), (int64_t)(N - n0) * (K / 2));
    const __amdgpu_buffer_rsrc_t rb_s = make_rsrc(SFB + (int64_t)n0 * (K / 16), (int64_t)(N - n0) * (K / 16));
    const Fp4GroupOffsets<BM, BN, NT> off(m0, M, n0, N, K, tid);
    const int64_t kbase = (int64_t)sb * kF16StageK;
    const int64_t k_end = min(K, kbase + (int64_t)nst * kF16StageK);
    const int ngroups = (nst + 1) / 2;
    // lane offset inside a 32-row fragment block (blocks never straddle a shift)
    const uint8_t* fra = smem + lr * kF16Pitch + g * 16;
    const uint8_t* frb = fra;

    Fp4Group<BM, BN, NT> cur;
    fp4_group_load<BM, BN, NT>(cur, ra_q, ra_s, rb_q, rb_s, off, kbase, k_end);
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
      fp4_group_load<BM, BN, NT>(nxt, ra_q, ra_s, rb_q, rb_s, off, kbase + (int64_t)(gi + 1) * kGroupK, k_end);
      __builtin_amdgcn_sched_barrier(0);  // keep the loads at the top of the group
      // stage 2gi (slot 0): dequantise stage 2gi+1 of this group into slot 1
      f16_stage_compute<BM, BN, WGM, WGN>(fra, frb, acc, cur, smem + kStage, tid, true, wm, wn);
      __syncthreads();
      // stage 2gi+1 (slot 1): dequantise stage 0 of the next group into slot 0.
      // With an odd stage count the last one reads zeros (its K range lies past
      // k_end, so its codes and scales were loaded as zero) and adds nothing;
      // the loop keeps a single exit, which keeps register allocation sane.
      f16_stage_compute<BM, BN, WGM, WGN>(fra + kStage, frb + kStage, acc, nxt, smem, tid, false, wm, wn);
      __syncthreads();
      cur = nxt;
    }
  }

  // lane: output row m (its MFMA column), registers 4q..4q+3: columns n..n+3
  // (N % 4 == 0: the 4 columns are all in range or all out)
  const float alpha = alpha_ptr ? alpha_ptr[0] : 1.0f;
  if (splits == 1) {
    // bf16 tile through LDS (the stages are free after the K loop's last
    // barrier): each lane writes its 4-column runs into a row-major tile,
    // then every store instruction writes whole 16-byte-per-lane row segments
    // (BN * 2 contiguous bytes per row) instead of 64 scattered 8-byte pieces
    constexpr int kOutPitch = BN * 2 + 16;  // bytes per LDS row
    static_assert(BM * kOutPitch <= 2 * kStage, "output tile fits in the stage buffers");
#pragma unroll
    for (int i = 0; i < TM; i++) {
      const int r = wm * WM + i * 32 + lr;
#pragma unroll
      for (int j = 0; j < TN; j++)
#pragma unroll
        for (int q = 0; q < 4; q++) {
          const int c = wn * WN + j * 32 + 8 * q + 4 * g;
          *reinterpret_cast<uint2*>(smem + r * kOutPitch + c * 2) =
              make_uint2(pack_bf16x2(alpha * acc[i][j][4 * q], alpha * acc[i][j][4 * q + 1]),
                         pack_bf16x2(alpha * acc[i][j][4 * q + 2], alpha * acc[i][j][4 * q + 3]));
        }
    }
    __syncthreads();
    constexpr int kChunksPerRow = BN / 8;  // 16-byte chunks (8 columns)
    for (int idx = tid; idx < BM * kChunksPerRow; idx += NT) {
      const int r = idx / kChunksPerRow, c = (idx % kChunksPerRow) * 8;
      const int m = m0 + r, n = n0 + c;
      if (m < M && n < N)
        *reinterpret_cast<uint4*>(D + (int64_t)m * N + n) = *reinterpret_cast<const uint4*>(smem + r * kOutPitch + c * 2);
    }
    return;
  }
  // FP32 partial tile of split `split`, through LDS in kPasses row bands of
  // the same layout (16 bytes per lane per store, whole row segments)
  constexpr int kPartPitch = BN * 4 + 16;
  constexpr int kPasses = (BM * kPartPitch + 2 * kStage - 1) / (2 * kStage);
  constexpr int kBandRows = BM / kPasses;
  static_assert(kBandRows % 32 == 0 && kBandRows * kPartPitch <= 2 * kStage, "partial band fits in LDS");
  float* dst = part + (int64_t)split * M * N;
#pragma unroll
  for (int h = 0; h < kPasses; h++) {
    if (h > 0) __syncthreads();  // the previous band has been stored
#pragma unroll
    for (int i = 0; i < TM; i++) {
      const int r = wm * WM + i * 32;  // first row of the 32-row block (uniform)
      if (r / kBandRows != h) continue;
      const int rl = r - h * kBandRows + lr;
#pragma unroll
      for (int j = 0; j < TN; j++)
#pragma unroll
        for (int q = 0; q < 4; q++) {
          const int c = wn * WN + j * 32 + 8 * q + 4 * g;
          *reinterpret_cast<float4*>(smem + rl * kPartPitch + c * 4) =
              make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
        }
    }
    __syncthreads();
    constexpr int kChunksPerRow = BN / 4;  // 16-byte chunks (4 columns)
    for (int idx = tid; idx < kBandRows * kChunksPerRow; idx += NT) {
      const int rl = idx / kChunksPerRow, c = (idx % kChunksPerRow) * 4;
      const int m = m0 + h * kBandRows + rl, n = n0 + c;
      if (m < M && n < N)
        *reinterpret_cast<float4*>(dst + (int64_t)m * N + n) = *reinterpret_cast<const float4*>(smem + rl * kPartPitch + c * 4);
    }
  }
}

// D = bf16(alpha * sum_s part[s]), partials added in split order (deterministic).
__global__ void __launch_bounds__(256)
    splitk_reduce(const float* __restrict__ part, int splits, const float* __restrict__ alpha_ptr,
                  uint16_t* __restrict__ D, int64_t MN) {
  const float alpha = alpha_ptr ? alpha_ptr[0] : 1.0f;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < MN / 4; q += stride) {
    float4 acc = reinterpret_cast<const float4*>(part)[q];
    // up to 8 partials loaded before any is added (independent loads in flight),
    // then added in split order
    for (int s0 = 1; s0 < splits; s0 += 8) {
      float4 v[8];
#pragma unroll
      for (int j = 0; j < 8; j++)
        if (s0 + j < splits) v[j] = reinterpret_cast<const float4*>(part + (int64_t)(s0 + j) * MN)[q];
#pragma unroll
      for (int j = 0; j < 8; j++)
        if (s0 + j < splits) {
          acc.x += v[j].x;
          acc.y += v[j].y;
          acc.z += v[j].z;
          acc.w += v[j].w;
        }
    }
    reinterpret_cast<uint2*>(D)[q] = make_uint2(pack_bf16x2(alpha * acc.x, alpha * acc.y),
                                                pack_bf16x2(alpha * acc.z, alpha * acc.w));
  }
}

struct Plan {
  int bm, bn, splits;
};

// Tile shape and K split for an M x N x K problem on `cus` compute units.
// Estimated time = (rounds of work items) x (flops per item) / (measured rate
// of one workgroup of that tile shape) + the FP32 partial-sum traffic of a
// split and its reduce kernel.  Rates (TFLOP/s per workgroup, dequantise-once
// kernels on gfx950): 256x256 ~4.0, 256x128 ~3.0, 128x128 ~1.6 with two
// workgroups per CU.
// Test and measurement overrides, read on every call: BSFP4_NVFP4_TILE=256|128|
// 256x128 forces the tile shape, BSFP4_NVFP4_SPLITS=n the number of K splits.
const char* env_str(const char* name) { return getenv(name); }
int env_int(const char* name) {
  const char* e = getenv(name);
  return e ? atoi(e) : 0;
}

Plan plan_tiled(int64_t M, int64_t N, int64_t K, int cus, bool allow_256x128) {
  const int64_t stages = (K + 63) / 64;
  struct Cand { int bm, bn, per_cu; double rate; const char* name; };
  const Cand cands[3] = {{256, 256, 1, 4.0e12, "256"}, {256, 128, 1, 3.0e12, "256x128"},
                         {128, 128, 2, 1.6e12, "128"}};
  const char* force_tile = env_str("BSFP4_NVFP4_TILE");
  const int force_splits = env_int("BSFP4_NVFP4_SPLITS");
  Plan best{256, 256, 1};
  double best_t = 1e300;
  for (const Cand& c : cands) {
    if (force_tile && strcmp(force_tile, c.name)) continue;
    if (c.bm != c.bn && !allow_256x128) continue;
    const int64_t tiles = ((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn);
    for (int sp = 1; sp <= 8; sp++) {
      if (sp > 1 && stages / sp < 4) break;  // keep at least 4 stages (256 K values) per split
      if (force_splits > 0 && sp != std::min<int64_t>(force_splits, stages)) continue;
      const int64_t items = tiles * sp;
      const int64_t slots = (int64_t)cus * c.per_cu;
      const int64_t rounds = (items + slots - 1) / slots;
      double t = rounds * (2.0 * c.bm * c.bn * (double)K / sp) / c.rate;
      // partials written (coalesced, overlapping other tiles' compute) and read
      // back by the reduction: ~8 TB/s effective, measured
      if (sp > 1) t += (2.0 * sp * M * N * 4 + 2.0 * M * N) / 8.0e12 + 3e-6;
      if (t < best_t * 0.999) {
        best_t = t;
        best = Plan{c.bm, c.bn, sp};
      }
    }
  }
  return best;
}


}  // namespace

// 256x256 tiles: the dequantise-once kernel with 16 waves of 64x64 by default
// (four per SIMD, 128 VGPRs each: measured 2 % faster at 4096 x 4096 x 7168 than
// 8 waves of 128x64, which hide less of the LDS and barrier latency).
// BSFP4_NVFP4_KERNEL selects an alternative for measurements: "w8" (same
// kernel, 8 waves of 128x64), "lds4" (4 waves of 128x128), "reg8" / "reg4"
// (per-wave register dequantisation, 8 or 4 waves).
// The dequantise-once kernel addresses operands with 32-bit buffer offsets
// (M*K/2 and N*K/2 below 2^31); larger operands take the register-dequant
// kernel.
// variants 0, 1 and 4 are the dequantise-once kernel
static bool dequant_once(int v) { return v == 0 || v == 1 || v == 4; }

static int nvfp4_variant(int64_t M, int64_t N, int64_t K) {
  const char* e = getenv("BSFP4_NVFP4_KERNEL");
  int v = 0;
  if (e && !strcmp(e, "lds4")) v = 1;
  if (e && !strcmp(e, "reg8")) v = 2;
  if (e && !strcmp(e, "reg4")) v = 3;
  if (e && !strcmp(e, "w8")) v = 4;
  const int64_t lim = (int64_t)1 << 31;
  if (dequant_once(v) && (M * (K / 2) >= lim || N * (K / 2) >= lim)) v = 2;
  return v;
}

hipError_t launch_nvfp4_gemm(const uint8_t* A, const uint8_t* SFA, const uint8_t* B, const uint8_t* SFB,
                             const float* alpha, uint16_t* D, int64_t M, int64_t N, int64_t K,
                             void* ws, size_t ws_bytes, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  if (nvfp4_rows64_ok(M, N, K))
    return launch_nvfp4_rows64(A, SFA, B, SFB, alpha, D, M, N, K, static_cast<float*>(ws), ws_bytes, stream);
  if (M <= kSkinnyMaxM)
    return launch_skinny_nvfp4(A, SFA, B, SFB, alpha, D, M, N, K, static_cast<float*>(ws), stream);
  const int v = nvfp4_variant(M, N, K);
  Plan pl = plan_tiled(M, N, K, device_cu_count(), dequant_once(v));
  if (pl.splits > 1 && ws_bytes < (size_t)pl.splits * M * N * sizeof(float)) pl.splits = 1;
  float* part = static_cast<float*>(ws);
  const int tiles_m = (int)((M + pl.bm - 1) / pl.bm);
  const int tiles_n = (int)((N + pl.bn - 1) / pl.bn);
  const unsigned grid = (unsigned)(tiles_m * tiles_n * pl.splits);
#define BSFP4_ARGS A, SFA, B, SFB, alpha, D, (int)M, (int)N, K
  if (pl.bm == 256 && pl.bn == 256) {
    switch (v) {
      case 1: nvfp4_gemm_f16lds<256, 256, 2, 2><<<grid, 256, 0, stream>>>(BSFP4_ARGS, tiles_m, tiles_n, pl.splits, part); break;
      case 2: nvfp4_gemm_tiled<256, 256, 2, 4><<<grid, 512, 0, stream>>>(BSFP4_ARGS, tiles_n, pl.splits, part); break;
      case 3: nvfp4_gemm_tiled<256, 256, 2, 2><<<grid, 256, 0, stream>>>(BSFP4_ARGS, tiles_n, pl.splits, part); break;
      case 4: nvfp4_gemm_f16lds<256, 256, 2, 4><<<grid, 512, 0, stream>>>(BSFP4_ARGS, tiles_m, tiles_n, pl.splits, part); break;
      default: nvfp4_gemm_f16lds<256, 256, 4, 4><<<grid, 1024, 0, stream>>>(BSFP4_ARGS, tiles_m, tiles_n, pl.splits, part);
    }
  } else if (pl.bm == 256) {  // 256x128 (planned only for the dequantise-once kernels)
    nvfp4_gemm_f16lds<256, 128, 2, 2><<<grid, 256, 0, stream>>>(BSFP4_ARGS, tiles_m, tiles_n, pl.splits, part);
  } else {
    if (!dequant_once(v))
      nvfp4_gemm_tiled<128, 128, 2, 2><<<grid, 256, 0, stream>>>(BSFP4_ARGS, tiles_n, pl.splits, part);
    else
      nvfp4_gemm_f16lds<128, 128, 2, 2><<<grid, 256, 0, stream>>>(BSFP4_ARGS, tiles_m, tiles_n, pl.splits, part);
  }
#undef BSFP4_ARGS
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.splits == 1) return e;
  return launch_splitk_reduce(part, pl.splits, alpha, D, M * N, stream);
}

hipError_t launch_splitk_reduce(const float* part, int splits, const float* alpha, uint16_t* D, int64_t MN,
                                hipStream_t stream) {
  const int64_t q = MN / 4;
  const unsigned rgrid = (unsigned)((q + 255) / 256 > 16384 ? 16384 : (q + 255) / 256);
  splitk_reduce<<<rgrid < 1 ? 1 : rgrid, 256, 0, stream>>>(part, splits, alpha, D, MN);
  return hipGetLastError();
}

// Compute units of the current device, cached per device id (a fixed property
// of the device; 256 if the query fails or the id is out of the cache's range).
int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
  if (dev < 64) cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

size_t nvfp4_gemm_workspace(int64_t M, int64_t N, int64_t K) {
  if (nvfp4_rows64_ok(M, N, K)) return w4a16_rows64_workspace(M, N, K);
  if (M <= kSkinnyMaxM) return skinny_workspace(M, N, K, true);
  const Plan pl = plan_tiled(M, N, K, device_cu_count(), dequant_once(nvfp4_variant(M, N, K)));
  return pl.splits > 1 ? (size_t)pl.splits * M * N * sizeof(float) : 0;
}

}  // namespace bsfp4

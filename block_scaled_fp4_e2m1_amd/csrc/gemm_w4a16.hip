// GEMMs of more than 16 rows with NVFP4 weights on gfx950.
//
// W4A16: D = bf16(alpha * A @ dec(B)^T) with A bf16 [M, K], B NVFP4 (E2M1
// codes [N, K/2], one E4M3 scale per 16 K-elements [N, K/16]) and alpha the
// tensor-wide weight scale applied to the FP32 accumulator: the dense W4A16
// GEMM of the FlashInfer `mm_bf16_fp4` pages ("feat: sm100 cute_dsl w4a16
// gemm" and its follow-ups).  The row kernel further down also takes NVFP4
// activations (the W4A4 GEMM of "perf(gemm): optimize SM103 CuTe DSL mm_fp4
// kernel" at 24..128 rows).  Two kernels: the tiled kernel below for more than
// 128 rows (and 65..128 rows when K % 128 != 0), the row kernel for 17..128
// rows; 16 rows and fewer (and 17..64 rows when K % 128 != 0) use the
// weight-streaming kernels of gemm_skinny.hip.
//
// An E2M1 value times an E4M3 scale has at most 6 significant bits, so the
// dequantised weights are exact in bf16 and v_mfma_f32_32x32x16_bf16 forms the
// exact products with FP32 accumulation.
//
// Tiled kernel: one workgroup = 8 waves (1 x 8) on a 256 x 256 output tile,
// 256 x 32 per wave, so every B fragment is read and dequantised by exactly
// one wave (the A fragments, plain bf16, are read by all eight; measured
// 3-12 % faster at the projection shapes than 2 x 4 waves of 128 x 64); K in
// stages of 64 values.  A 3-slot LDS ring is filled by direct-to-LDS buffer
// loads issued by 4 loader waves: per stage the A rows (128 bytes of bf16,
// their 16-byte chunks XOR-swizzled by row so that the fragment reads are
// conflict-free), the B code rows (32 bytes, chunk order swapped on alternate
// 8-row blocks) and the B scale bytes (4 per row).  Each wave reads its A
// fragments as bf16 and dequantises its B fragments in registers.  B is the
// MFMA's first operand, so a lane ends with runs of 4 consecutive output
// columns of one row; the tile leaves through LDS in row bands (bf16 output,
// or FP32 partials of a K split that splitk_reduce sums in split order).
#include <algorithm>
#include <cstdlib>
#include <type_traits>

#include "device_common.h"
#include "launchers.h"
#include "lds_dma.h"

namespace bsfp4 {
namespace {

constexpr int kBM = 256, kBN = 256;
constexpr int kWGM = 1, kWGN = 8;
constexpr int kNT = 64 * kWGM * kWGN;
constexpr int kWM = kBM / kWGM, kWN = kBN / kWGN;
constexpr int kTM = kWM / 32, kTN = kWN / 32;
constexpr int kSK = 64;                    // K values per stage
constexpr int kARow = kSK * 2;             // bytes of one A row per stage (bf16)
constexpr int kBRow = kSK / 2;             // bytes of one B code row per stage
constexpr int kSRow = kSK / 16;            // scale bytes of one B row per stage
constexpr int kA = kBM * kARow;
constexpr int kBq = kBN * kBRow;
constexpr int kBs = kBN * kSRow;
constexpr int kStage = kA + kBq + kBs;
constexpr int kRing = 3;
constexpr int kLoad = 4;                   // loader waves
constexpr int kAI = kA / 1024 / kLoad;     // A loads (1 KB each) per loader wave per stage
constexpr int kBqI = kBq / 1024 / kLoad;   // B code loads (1 KB each)
constexpr int kBsI = kBs / 256 / kLoad;    // B scale loads (256 B each)
constexpr int kL = kAI + kBqI + kBsI;
static_assert(kAI * kLoad * 1024 == kA && kBqI * kLoad * 1024 == kBq && kBsI * kLoad * 256 == kBs,
              "loads cover the stage exactly");
static_assert(kRing * kStage <= 160 * 1024, "ring fits in LDS");

// 16-byte chunk positions: A rows hold 8 chunks, B code rows 2
__device__ __forceinline__ int swz_a(int r, int c) { return c ^ ((r ^ (r >> 3)) & 7); }
__device__ __forceinline__ int swz_b(int r, int c) { return c ^ ((r >> 3) & 1); }

__global__ void __launch_bounds__(kNT, 1)
    w4a16_tiled(const uint16_t* __restrict__ A, const uint8_t* __restrict__ B, const uint8_t* __restrict__ SFB,
                const float* __restrict__ alpha_ptr, uint16_t* __restrict__ D, int M, int N, int K, int tiles_m,
                int tiles_n, int splits, float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kRing * kStage];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / kWGN, wn = wave % kWGN;
  const int lr = lane & 31, g = lane >> 5;

  // work item -> (tile, split): consecutive items on one XCD, tiles in bands of
  // 4 tile rows so that an XCD's items share few A and B panels
  const int items = tiles_m * tiles_n * splits;
  int item = blockIdx.x;
  if (items % 8 == 0) item = (int)(blockIdx.x % 8) * (items / 8) + (int)(blockIdx.x / 8);
  const int split = item % splits;
  const int tile = item / splits;
  const int band_tiles = 4 * tiles_n;
  const int band = tile / band_tiles, in_band = tile % band_tiles;
  const int band_rows = min(4, tiles_m - band * 4);
  const int m0 = (band * 4 + in_band % band_rows) * kBM;
  const int n0 = (in_band / band_rows) * kBN;
  const int total = K / kSK;
  const int sb = (int)((int64_t)total * split / splits);
  const int nst = (int)((int64_t)total * (split + 1) / splits) - sb;

  v16f acc[kTM][kTN];
#pragma unroll
  for (int i = 0; i < kTM; i++)
#pragma unroll
    for (int j = 0; j < kTN; j++) acc[i][j] = v16f{};

  // ---- per-lane load offsets (the stage's K offset goes in the SGPR offset)
  const bool loader = wave < kLoad;
  const int lw = loader ? wave : 0;
  const v4u32 ra = make_rsrc4(A, (int64_t)M * K * 2);
  const v4u32 rq = make_rsrc4(B, (int64_t)N * (K / 2));
  const v4u32 rs = make_rsrc4(SFB, (int64_t)N * (K / 16));
  uint32_t va[kAI], vq[kBqI], vs[kBsI];
#pragma unroll
  for (int j = 0; j < kAI; j++) {
    const int q = lw * kAI + j;
    const int row = q * 8 + (lane >> 3);
    const int c = swz_a(row, lane & 7);  // swz_a is its own inverse
    va[j] = m0 + row < M ? (uint32_t)((m0 + row) * (K * 2) + c * 16) : kBufOOB;
  }
#pragma unroll
  for (int j = 0; j < kBqI; j++) {
    const int q = lw * kBqI + j;
    const int row = q * 32 + (lane >> 1);
    const int c = swz_b(row, lane & 1);
    vq[j] = n0 + row < N ? (uint32_t)((n0 + row) * (K / 2) + c * 16) : kBufOOB;
  }
#pragma unroll
  for (int j = 0; j < kBsI; j++) {
    const int row = (lw * kBsI + j) * 64 + lane;
    vs[j] = n0 + row < N ? (uint32_t)((n0 + row) * (K / 16)) : kBufOOB;
  }
  const uint32_t lds0 = lds_offset(smem);
  auto issue = [&](int st) {
    const int k0 = (sb + st) * kSK;
    const uint32_t base = lds0 + (uint32_t)((st % kRing) * kStage);
#pragma unroll
    for (int j = 0; j < kAI; j++)
      buf_lds16(uniform4(ra), va[j], (uint32_t)(k0 * 2),
                (uint32_t)__builtin_amdgcn_readfirstlane((int)(base + (wave * kAI + j) * 1024)));
#pragma unroll
    for (int j = 0; j < kBqI; j++)
      buf_lds16(uniform4(rq), vq[j], (uint32_t)(k0 / 2),
                (uint32_t)__builtin_amdgcn_readfirstlane((int)(base + kA + (wave * kBqI + j) * 1024)));
#pragma unroll
    for (int j = 0; j < kBsI; j++)
      buf_lds4(uniform4(rs), vs[j], (uint32_t)(k0 / 16),
               (uint32_t)__builtin_amdgcn_readfirstlane((int)(base + kA + kBq + (wave * kBsI + j) * 256)));
  };

  if (nst > 0) {
    if (loader)
      for (int st = 0; st < kRing - 1 && st < nst; st++) issue(st);
    for (int s = 0; s < nst; s++) {
      if (loader) {
        if (s + 1 < nst) wait_vmcnt<kL>();  // kRing - 1 = 2 stages were in flight
        else wait_vmcnt<0>();
      }
      __builtin_amdgcn_s_barrier();  // stage s visible; every wave is past stage s-1
      if (loader && s + kRing - 1 < nst) issue(s + kRing - 1);
      const uint8_t* st = smem + (s % kRing) * kStage;
      const uint8_t* sa = st;
      const uint8_t* sq = st + kA;
      const uint8_t* ss = st + kA + kBq;
      // this lane's B rows: its 4 code words (K values 16kk + 8g .. +7, word
      // 2kk + g of the row) and the row's 4 scale bytes
      uint32_t bw[kTN][4], bsc[kTN];
#pragma unroll
      for (int jn = 0; jn < kTN; jn++) {
        const int r = wn * kWN + jn * 32 + lr;
        const uint4 c0 = *reinterpret_cast<const uint4*>(sq + r * kBRow + swz_b(r, 0) * 16);
        const uint4 c1 = *reinterpret_cast<const uint4*>(sq + r * kBRow + swz_b(r, 1) * 16);
        bw[jn][0] = g ? c0.y : c0.x;
        bw[jn][1] = g ? c0.w : c0.z;
        bw[jn][2] = g ? c1.y : c1.x;
        bw[jn][3] = g ? c1.w : c1.z;
        bsc[jn] = *reinterpret_cast<const uint32_t*>(ss + r * kSRow);
      }
#pragma unroll
      for (int kk = 0; kk < kSK / 16; kk++) {
        // K values 16kk + 8g .. +7 of the stage: code word 2kk + g, scale byte kk
        v8bf fb[kTN];
#pragma unroll
        for (int jn = 0; jn < kTN; jn++)
          fb[jn] = dq8_bf16(bw[jn][kk], e4m3_to_f32((bsc[jn] >> (8 * kk)) & 0xFFu));
#pragma unroll
        for (int i = 0; i < kTM; i++) {
          const int r = wm * kWM + i * 32 + lr;
          const v8bf fa = *reinterpret_cast<const v8bf*>(sa + r * kARow + swz_a(r, 2 * kk + g) * 16);
#pragma unroll
          for (int jn = 0; jn < kTN; jn++)
            acc[i][jn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[jn], fa, acc[i][jn], 0, 0, 0);
        }
      }
    }
  }
  __syncthreads();  // the ring is free: the tile leaves through it

  // acc[i][jn][4q + t] = row wm*WM + 32i + lr, column wn*WN + 32jn + 8q + 4g + t
  const float alpha = alpha_ptr ? alpha_ptr[0] : 1.0f;
  auto out_bands = [&](auto elem) {
    constexpr int kE = decltype(elem)::value;  // bytes per output element
    constexpr int kPitch = kBN * kE + 16;
    constexpr int kRingBytes = kRing * kStage;
    constexpr int kPasses = kBM * kPitch <= kRingBytes         ? 1
                            : (kBM / 2) * kPitch <= kRingBytes ? 2
                            : (kBM / 4) * kPitch <= kRingBytes ? 4
                                                               : 8;
    constexpr int kBand = kBM / kPasses;
    static_assert(kBand % 32 == 0 && kBand * kPitch <= kRing * kStage, "band fits in the ring");
    float* dst_part = part + (int64_t)split * M * N;
#pragma unroll
    for (int h = 0; h < kPasses; h++) {
      if (h > 0) __syncthreads();
#pragma unroll
      for (int i = 0; i < kTM; i++) {
        const int r = wm * kWM + i * 32;
        if (r / kBand != h) continue;
        uint8_t* row = smem + (r - h * kBand + lr) * kPitch;
#pragma unroll
        for (int jn = 0; jn < kTN; jn++)
#pragma unroll
          for (int q = 0; q < 4; q++) {
            const int c = wn * kWN + jn * 32 + 8 * q + 4 * g;
            if constexpr (kE == 4)
              *reinterpret_cast<float4*>(row + c * 4) =
                  make_float4(acc[i][jn][4 * q], acc[i][jn][4 * q + 1], acc[i][jn][4 * q + 2], acc[i][jn][4 * q + 3]);
            else
              *reinterpret_cast<uint2*>(row + c * 2) =
                  make_uint2(pack_bf16x2(alpha * acc[i][jn][4 * q], alpha * acc[i][jn][4 * q + 1]),
                             pack_bf16x2(alpha * acc[i][jn][4 * q + 2], alpha * acc[i][jn][4 * q + 3]));
          }
      }
      __syncthreads();
      constexpr int kChunks = kBN * kE / 16;  // 16-byte chunks per row
      for (int idx = tid; idx < kBand * kChunks; idx += kNT) {
        const int rl = idx / kChunks, cb = (idx % kChunks) * 16;
        const int m = m0 + h * kBand + rl, n = n0 + cb / kE;
        if (m >= M || n >= N) continue;
        const uint4 v = *reinterpret_cast<const uint4*>(smem + rl * kPitch + cb);
        if constexpr (kE == 4)
          *reinterpret_cast<uint4*>(dst_part + (int64_t)m * N + n) = v;
        else
          *reinterpret_cast<uint4*>(D + (int64_t)m * N + n) = v;
      }
    }
  };
  if (splits == 1)
    out_bands(std::integral_constant<int, 2>{});
  else
    out_bands(std::integral_constant<int, 4>{});
}


// ---------------------------------------------------------------------------
// Row GEMM for up to 128 rows (W4A16 from 17, NVFP4 from 24 rows; fewer rows
// use the kernels of gemm_skinny.hip), W4A16 (AKIND 1: bf16 activations, bf16 MFMA) or NVFP4 W4A4
// (AKIND 0: NVFP4 activations dequantised to fp16, fp16 MFMA; E2M1 x E4M3
// values are exact in either type): one workgroup = all BM = 64 or 128 rows x
// 128 output columns x one K range, 8 waves = 2 column halves x 4 K quarters
// of every stage: a wave owns 64 columns x BM rows (4 x BM/16
// v_mfma_f32_16x16x32 tiles) for 32 of the stage's 128 K values, so every
// weight value is dequantised exactly once per workgroup and each weight
// fragment feeds BM/16 MFMAs; the four K quarters are summed in LDS at the
// end, in quarter order, 64 rows at a time.  The weight stream is what costs
// at these shapes; the activations (at most 128 rows) stay L2-resident and
// are re-read once per 128-column block.
//   * codes move stage by stage through LDS rings of 4 slots (3 for 128 rows,
//     whose activation stages are twice as large), three (two) stages ahead
//     of the one in use, so each stage waits only for its own loads and the
//     MFMAs follow the stream: per stage the weight codes (one load per wave:
//     16 rows x 64 bytes into [row][64 B], the 16-byte piece p of row r at
//     position p ^ ((r >> 2) & 3), so the MFMA's 4-byte reads are
//     conflict-free) and the activations.  Measured for W4A16 at 64 x 4096 x
//     7168 cold (both kernels, events): the range's weights issued before the
//     first stage 22.7 us, 5 / 4 / 3 stages ahead 22.4 / 21.7 / 21.4 us (the
//     first of these is 16.6 us of this kernel in a rocprofv3 trace, against
//     17.7 us when the range was copied in long row segments ahead of
//     everything);
//   * the scales (8 bytes per row and stage) come in double-buffered chunks of
//     eight stages, 64 bytes per row (16 lanes of 4 bytes per row, 4 rows per
//     load, dwords swizzled within the row so that the scale reads are
//     conflict-free): chunk 0 before the first stage, chunk k with the codes
//     of stage 8k - 1.  One load of 8 bytes per row and stage measured 1.7 us
//     slower at 64 x 4096 x 7168 (each such load touches 32 rows), unswizzled
//     chunks 0.4 us slower (8-way bank conflicts);
//   * bf16 activations: BM rows x 256 bytes a stage, the 16-byte chunk x of
//     row r at position x ^ (r & 15) (conflict-free fragment reads), BM/32
//     loads per wave;
//   * NVFP4 activations: the stage's BM rows x 64 code bytes (one load per
//     wave below BM/16; the scale chunks by all waves) are dequantised once
//     per workgroup, one stage ahead of the MFMAs, into a 2-slot fp16 buffer
//     laid out like the bf16 stages (each thread BM/64 16-value blocks: two
//     code words and one scale byte each), so stage s waits for its weights
//     and for the activations of stage s + 1;
//   * K ranges of one column block are summed by splitk_reduce in range order;
//     a range may hold any number of stages (the K split is planned by rounds
//     of workgroups, rows64_splits).
constexpr int kRBN = 128, kRNT = 512;
constexpr int kRSK = 128;                     // K values per stage
constexpr int kRW = kRBN * 64;                 // weight codes of a stage [128 rows][64 B]
constexpr int kRChunk = 8;                     // stages per scale chunk
constexpr int kRScW = kRBN * 8 * kRChunk;      // weight scales of a chunk [128 rows][64 B]
constexpr int kRHalf = 64;                     // rows of one quarter-sum pass
constexpr int kRedBytes = 4 * kRHalf * (kRBN + 4) * 4;  // the four K quarters' FP32 tiles of 64 rows

// LDS plan of the BM-row kernel (BM = 64 or 128): RING stages (4, or 3 for
// 128 rows) of activations (bf16: BM x 256 B; NVFP4: 2 fp16 stages and a ring
// of BM x 64 code bytes) and of weight codes, and two scale chunks.
template <int BM>
struct RowsGeo {
  static constexpr int kRing = BM == 64 ? 4 : 3;
  static constexpr int kA = BM * kRSK * 2;     // bf16 / fp16 activations of a stage
  static constexpr int kAq = BM * 64;          // NVFP4 activation codes of a stage
  static constexpr int kScA = BM * 8 * kRChunk;  // NVFP4 activation scales of a chunk [BM rows][64 B]
  static constexpr int kActBytes = kRing * kA;
  static_assert(2 * kA + kRing * kAq <= kActBytes, "NVFP4 activation buffers fit");
  static constexpr int kScBase = kActBytes + kRing * kRW;
  static constexpr int kLoadBytes = kScBase + 2 * (kRScW + kScA);
  static constexpr int kSmem = kLoadBytes > kRedBytes ? kLoadBytes : kRedBytes;
  static_assert(kSmem <= 160 * 1024, "LDS");
};

template <int AKIND, int BM>
__global__ void __launch_bounds__(kRNT)
    rows64_gemm(const void* __restrict__ Aptr, const uint8_t* __restrict__ SFA, const uint8_t* __restrict__ B,
                const uint8_t* __restrict__ SFB, const float* __restrict__ alpha_ptr, uint16_t* __restrict__ D,
                int M, int N, int K, int splits, float* __restrict__ part) {
  constexpr bool kFp4A = AKIND == 0;
  using G = RowsGeo<BM>;
  constexpr int kRing = G::kRing, kRA = G::kA, kRAq = G::kAq, kRScA = G::kScA;
  constexpr int kTM = BM / 16;  // 16-row MFMA tiles of a wave
  __shared__ __attribute__((aligned(16))) uint8_t smem[G::kSmem];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int split = blockIdx.x % splits;
  const int n0 = (blockIdx.x / splits) * kRBN;
  const int total = K / kRSK;
  const int sb = (int)((int64_t)total * split / splits);
  const int nst = (int)((int64_t)total * (split + 1) / splits) - sb;
  const int k_lo = sb * kRSK;
  uint8_t* const sw = smem + G::kActBytes;  // [slot][codes 128 x 64 B]
  uint8_t* const saq = smem + 2 * kRA;      // NVFP4: [slot][codes BM x 64 B]
  uint8_t* const ssc = smem + G::kScBase;   // [chunk % 2][W scales 128 x 64 B | A scales BM x 64 B]
  const v4u32 ra = make_rsrc4(Aptr, kFp4A ? (int64_t)M * (K / 2) : (int64_t)M * K * 2);
  const v4u32 rq = make_rsrc4(B, (int64_t)N * (K / 2));
  const v4u32 rs = make_rsrc4(SFB, (int64_t)N * (K / 16));
  auto lds_u = [](const void* p) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_offset(p)); };
  auto soff = [](int v) { return (uint32_t)__builtin_amdgcn_readfirstlane(v); };

  // ---- per-lane offsets (the stage's K offset goes in the SGPR offset)
  // weight codes: rows 16 wave + lane / 4, logical piece (lane & 3) ^ ((row >> 2) & 3)
  // of the stage's 64 bytes at LDS position lane & 3
  const int wrow = 16 * wave + (lane >> 2);
  const uint32_t vw = n0 + wrow < N
                          ? (uint32_t)((n0 + wrow) * (K / 2) + k_lo / 2 + 16 * ((lane & 3) ^ ((wrow >> 2) & 3)))
                          : kBufOOB;
  // scale chunks: load j (0..3) of wave w covers weight rows 4 (4 w + j) +
  // lane / 16, NVFP4 activation load j (0..BM/32-1) rows 4 (BM/32 w + j) +
  // lane / 16; dword d of the chunk's 64 bytes of row r lands at position
  // d ^ (r & 15) of the row, so the 16 rows that one scale read spans hit
  // distinct banks
  constexpr int kAsc = BM / 32;  // activation-scale loads per wave and chunk (NVFP4)
  uint32_t vws[4], vas[kAsc];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int wr = 4 * (4 * wave + j) + (lane >> 4);
    vws[j] = n0 + wr < N ? (uint32_t)((n0 + wr) * (K / 16) + k_lo / 16 + 4 * ((lane & 15) ^ (wr & 15))) : kBufOOB;
  }
#pragma unroll
  for (int j = 0; j < kAsc; j++) {
    const int ar = 4 * (kAsc * wave + j) + (lane >> 4);
    vas[j] = ar < M ? (uint32_t)(ar * (K / 16) + k_lo / 16 + 4 * ((lane & 15) ^ (ar & 15))) : kBufOOB;
  }
  // byte `byte` of row r's 64 chunk bytes (dword swizzle above)
  auto sc_at = [](int r, int byte) { return r * 64 + (((byte >> 2) ^ (r & 15)) << 2) + (byte & 3); };
  // activations: NVFP4 codes, waves w < BM/16: rows 16 w + lane / 4, 16-byte
  // piece lane & 3 of the stage's 64 bytes; bf16, BM/32 loads per wave: rows
  // 4 (BM/32 w + j) + lane / 16, the 16-byte chunk landing at position lane & 15
  constexpr int kAb = BM / 32;  // bf16 activation loads per wave and stage
  uint32_t va[kFp4A ? 1 : kAb];
  if constexpr (kFp4A) {
    const int r = 16 * wave + (lane >> 2);
    va[0] = (wave < BM / 16 && r < M) ? (uint32_t)(r * (K / 2) + k_lo / 2 + 16 * (lane & 3)) : kBufOOB;
  } else {
#pragma unroll
    for (int j = 0; j < kAb; j++) {
      const int r = 4 * (kAb * wave + j) + (lane >> 4);
      const int x = (lane & 15) ^ (r & 15);  // global chunk landing at position lane & 15
      va[j] = r < M ? (uint32_t)(r * (K * 2) + x * 16) : kBufOOB;
    }
  }
  // This wave's loads of one stage, in issue order: NVFP4 the activation
  // codes (waves below BM/16) then the weight codes; bf16 weight codes then
  // BM/32 activation loads.  A scale chunk is cl loads: 4 of weight scales and
  // for NVFP4 BM/32 of activation scales.
  const int n_act = kFp4A ? (wave < BM / 16 ? 1 : 0) : kAb;
  const int per_stage = n_act + 1;
  constexpr int cl = 4 + (kFp4A ? kAsc : 0);
  const int nchunks = (nst + kRChunk - 1) / kRChunk;
  auto issue_chunk = [&](int k) {
    uint8_t* buf = ssc + (k & 1) * (kRScW + kRScA);
#pragma unroll
    for (int j = 0; j < 4; j++) buf_lds4(rs, vws[j], soff(64 * k), lds_u(buf + (4 * wave + j) * 256));
    if constexpr (kFp4A) {
      const v4u32 ras = make_rsrc4(SFA, (int64_t)M * (K / 16));
#pragma unroll
      for (int j = 0; j < kAsc; j++)
        buf_lds4(ras, vas[j], soff(64 * k), lds_u(buf + kRScW + (kAsc * wave + j) * 256));
    }
  };
  auto issue_w = [&](int st) {
    buf_lds16(rq, vw, soff(st * 64), lds_u(sw + (st % kRing) * kRW + wave * 1024));
  };
  auto issue = [&](int st) {
    if constexpr (kFp4A) {
      if (wave < BM / 16) buf_lds16(ra, va[0], soff(st * 64), lds_u(saq + (st % kRing) * kRAq + wave * 1024));
      issue_w(st);
    } else {
      issue_w(st);
      uint8_t* base = smem + (st % kRing) * kRA;
      const uint32_t k0 = soff((k_lo + st * kRSK) * 2);
#pragma unroll
      for (int j = 0; j < kAb; j++) buf_lds16(ra, va[j], k0, lds_u(base + (kAb * wave + j) * 1024));
    }
  };
  // NVFP4: dequantise stage st's activation codes into fp16 slot st % 2; a
  // thread takes BM/64 (row, 16-value block) items, chunks 2b and 2b + 1 of the row
  auto dequant_a = [&](int st) {
    const uint8_t* asc = ssc + ((st / kRChunk) & 1) * (kRScW + kRScA) + kRScW;
#pragma unroll
    for (int i = 0; i < BM / 64; i++) {
      const int it = tid + kRNT * i, r = it >> 3, b = it & 7;
      const uint2 w = *reinterpret_cast<const uint2*>(saq + (st % kRing) * kRAq + r * 64 + 8 * b);
      const _Float16 s = e4m3_to_f16(asc[sc_at(r, (st % kRChunk) * 8 + b)]);
      uint8_t* row = smem + (st & 1) * kRA + r * 256;
      *reinterpret_cast<v8h*>(row + (((2 * b) ^ (r & 15)) * 16)) = dq8_f16(w.x, s);
      *reinterpret_cast<v8h*>(row + (((2 * b + 1) ^ (r & 15)) * 16)) = dq8_f16(w.y, s);
    }
  };
  // This wave's issue order: chunk 0, stages 0 .. kAhead - 1, then at stage s
  // the loads of stage s + kAhead, followed by chunk k when s + kAhead ==
  // 8k - 1.  Loads complete in order; waiting for "issued - 1 - index"
  // outstanding means the load at that index has landed.
  constexpr int kAhead = kRing - 1;
  auto chunks_before = [&](int st) { return min(st / kRChunk, nchunks - 1); };  // chunks k >= 1 before stage st
  auto last_of_stage = [&](int st) { return cl - 1 + per_stage * (st + 1) + cl * chunks_before(st); };
  auto last_of_chunk = [&](int k) { return k == 0 ? cl - 1 : last_of_stage(kRChunk * k - 1) + cl; };
  auto issued_before = [&](int s) {  // loads issued before stage s's wait
    const int g = min(nst, s + kAhead);
    return cl + per_stage * g + cl * min(g / kRChunk, nchunks - 1);
  };
  issue_chunk(0);
  for (int st = 0; st < min(nst, kAhead); st++) issue(st);
  if constexpr (kFp4A) {
    // the activation codes and scales of stage 0
    wait_vmcnt_upto(issued_before(0) - 1 - (n_act > 0 ? last_of_stage(0) - per_stage + n_act : last_of_chunk(0)));
    __builtin_amdgcn_s_barrier();
    dequant_a(0);
  }

  // wave = (column half h: 64 columns, K quarter q of every stage: 32 values);
  // lane (c, g) of the 16x16x32 MFMAs: weight row / activation row c, K 8g..8g+7
  const int c = lane & 15, g = lane >> 4;
  const int h = wave & 1, q = wave >> 1;
  v4f acc[4][kTM];
#pragma unroll
  for (int j = 0; j < 4; j++)
#pragma unroll
    for (int t = 0; t < kTM; t++) acc[j][t] = v4f{};
  for (int s = 0; s < nst; s++) {
    // this wave's loads of stage s (and so its scale chunk); NVFP4 also the
    // activation codes of stage s + 1 (waves that load them) or else the
    // scale chunk of stage s + 1
    int last = last_of_stage(s);
    if (kFp4A && s + 1 < nst)
      last = n_act > 0 ? last_of_stage(s + 1) - per_stage + n_act : max(last, last_of_chunk((s + 1) / kRChunk));
    wait_vmcnt_upto(issued_before(s) - 1 - last);
    __builtin_amdgcn_s_barrier();  // stage s visible everywhere; every wave is past stage s-1
    if (s + kAhead < nst) {
      issue(s + kAhead);
      if ((s + kAhead) % kRChunk == kRChunk - 1 && s + kAhead + 1 < nst) issue_chunk((s + kAhead + 1) / kRChunk);
    }
    if constexpr (kFp4A) {
      if (s + 1 < nst) dequant_a(s + 1);  // read after the barrier at stage s + 1
    }
    const uint8_t* sa = smem + (kFp4A ? (s & 1) : (s % kRing)) * kRA;
    v8h fh[kTM];
    v8bf fa[kTM];
#pragma unroll
    for (int t = 0; t < kTM; t++) {
      const int r = 16 * t + c;
      const uint4 v = *reinterpret_cast<const uint4*>(sa + r * 256 + (((4 * q + g) ^ (r & 15)) * 16));
      if constexpr (kFp4A)
        fh[t] = __builtin_bit_cast(v8h, v);
      else
        fa[t] = __builtin_bit_cast(v8bf, v);
    }
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int col = 64 * h + 16 * j + c;
      // K values 32q + 8g .. +7 of the stage: code word 4q + g, scale byte 2q + g/2
      const uint32_t word = *reinterpret_cast<const uint32_t*>(sw + (s % kRing) * kRW + col * 64 +
                                                               ((q ^ ((col >> 2) & 3)) * 16) + 4 * g);
      const uint32_t sbw = ssc[((s / kRChunk) & 1) * (kRScW + kRScA) + sc_at(col, (s % kRChunk) * 8 + 2 * q + (g >> 1))];
      if constexpr (kFp4A) {
        const v8h fb = dq8_f16(word, e4m3_to_f16(sbw));
#pragma unroll
        for (int t = 0; t < kTM; t++) acc[j][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fb, fh[t], acc[j][t], 0, 0, 0);
      } else {
        const v8bf fb = dq8_bf16(word, e4m3_to_f32(sbw));
#pragma unroll
        for (int t = 0; t < kTM; t++) acc[j][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb, fa[t], acc[j][t], 0, 0, 0);
      }
    }
  }
  // ---- sum the four K quarters in LDS (in quarter order), 64 rows at a time, then store
  constexpr int kRedPitch = kRBN + 4;  // floats per row of one quarter's 64 x 128 tile
  static_assert(kRedBytes == 4 * kRHalf * kRedPitch * 4 && kRedBytes <= G::kSmem, "quarter tiles fit");
  float* red = reinterpret_cast<float*>(smem);
  const float alpha = alpha_ptr ? alpha_ptr[0] : 1.0f;
#pragma unroll
  for (int hh = 0; hh < BM / kRHalf; hh++) {
    __syncthreads();  // LDS is free (the ring, or the previous half's tiles)
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int t = 0; t < 4; t++)
        *reinterpret_cast<float4*>(red + (q * kRHalf + 16 * t + c) * kRedPitch + 64 * h + 16 * j + 4 * g) =
            make_float4(acc[j][4 * hh + t][0], acc[j][4 * hh + t][1], acc[j][4 * hh + t][2], acc[j][4 * hh + t][3]);
    __syncthreads();
    for (int idx = tid; idx < kRHalf * kRBN / 4; idx += kRNT) {  // 4 consecutive outputs per item
      const int ml = idx / (kRBN / 4), nl = (idx % (kRBN / 4)) * 4;
      const int m = kRHalf * hh + ml, n = n0 + nl;
      if (m >= M || n >= N) continue;
      float4 v = *reinterpret_cast<const float4*>(red + ml * kRedPitch + nl);
#pragma unroll
      for (int qq = 1; qq < 4; qq++) {
        const float4 u = *reinterpret_cast<const float4*>(red + (qq * kRHalf + ml) * kRedPitch + nl);
        v.x += u.x;
        v.y += u.y;
        v.z += u.z;
        v.w += u.w;
      }
      if (splits == 1)
        *reinterpret_cast<uint2*>(D + (int64_t)m * N + n) =
            make_uint2(pack_bf16x2(alpha * v.x, alpha * v.y), pack_bf16x2(alpha * v.z, alpha * v.w));
      else
        *reinterpret_cast<float4*>(part + ((int64_t)split * M + m) * N + n) = v;
    }
  }
}

// K split of the row kernel: the number of K ranges that minimises an
// estimate of the time in units of one stage (~0.6 us, measured cold): rounds
// of workgroups (one per CU) x (stages per range + ~3 for the set-up and the
// quarter sum), plus for a split the FP32 partials written and read back (M x N
// x 8 bytes per range at ~5 TB/s) and the reduce launch (~6).  Measurement
// override BSFP4_ROWS64_SPLITS=n.
constexpr int64_t kRMaxRows = 128;     // rows the kernel takes (64-row form up to 64, 128-row form above)
constexpr int64_t kRW4A16Rows = 128;   // default upper limits of the row kernel per activation kind
constexpr int64_t kRNvfp4Rows = 128;
int rows64_splits(int64_t M, int64_t N, int64_t K, int cus) {
  const int64_t tiles = (N + kRBN - 1) / kRBN, total = K / kRSK;
  if (total < 1) return 0;
  const char* e = getenv("BSFP4_ROWS64_SPLITS");
  if (e && atoi(e) > 0) return (int)std::min<int64_t>(atoi(e), total);
  constexpr double kStageUs = 0.6, kBytesPerUs = 5.0e6;
  int best = 1;
  double best_t = 1e300;
  for (int64_t sp = 1; sp <= std::min<int64_t>(total, 64); sp++) {
    const int64_t rounds = (tiles * sp + cus - 1) / cus;
    double t = (double)rounds * ((total + sp - 1) / sp + 3);
    if (sp > 1) t += 8.0 * sp * M * N / kBytesPerUs / kStageUs + 6;
    if (t < best_t * 0.999) {
      best_t = t;
      best = (int)sp;
    }
  }
  return best;
}

int w4a16_splits(int64_t M, int64_t N, int64_t K, int cus) {
  const int64_t tiles = ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
  const int64_t stages = K / kSK;
  int s = 1;
  while (s < 8 && tiles * (s + 1) <= cus && stages / (s + 1) >= 8) s++;
  return s;
}


}  // namespace

bool w4a16_tiled_ok(int64_t M, int64_t N, int64_t K) {
  const int64_t lim = (int64_t)1 << 31;
  return M > kSkinnyMaxM && K % kSK == 0 && M * K * 2 < lim && N * (K / 2) < lim;
}

size_t w4a16_tiled_workspace(int64_t M, int64_t N, int64_t K) {
  const int s = w4a16_splits(M, N, K, device_cu_count());
  return s > 1 ? (size_t)s * M * N * sizeof(float) : 0;
}

hipError_t launch_w4a16_tiled(const uint16_t* A, const uint8_t* B, const uint8_t* SFB, const float* alpha,
                              uint16_t* D, int64_t M, int64_t N, int64_t K, float* part, size_t part_bytes,
                              hipStream_t stream) {
  int splits = w4a16_splits(M, N, K, device_cu_count());
  if (splits > 1 && (part == nullptr || part_bytes < (size_t)splits * M * N * sizeof(float))) splits = 1;
  const int tiles_m = (int)((M + kBM - 1) / kBM), tiles_n = (int)((N + kBN - 1) / kBN);
  const unsigned grid = (unsigned)(tiles_m * tiles_n * splits);
  w4a16_tiled<<<grid, kNT, 0, stream>>>(A, B, SFB, alpha, D, (int)M, (int)N, (int)K, tiles_m, tiles_n, splits,
                                        part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  return launch_splitk_reduce(part, splits, alpha, D, M * N, stream);
}

}  // namespace bsfp4

namespace bsfp4 {

// Used for 17..128 rows.  Measured cold at N = 4096, K = 7168 (both kernels,
// events) against the split-K small-M kernels: M = 16 17.6 / 16.9 us (so 16
// and fewer rows keep those), M = 17 17.8 / 18.7, M = 32 19.2 / 20.4; at the
// projection shapes (M = 32; N x K = 6656 x 19968 / 19968 x 6656) 46.8 /
// 49.4 us, where K ranges of up to 8 stages took 67.8 / 65.6 us.  The
// 128-row form against the 256 x 256 tiled kernel: M = 65 / 96 / 128 at
// 4096 x 7168 24.5 / 25.4 / 26.5 against 36.1 / 36.5 / 37.5 us, M = 128 at
// the projection shapes 68.4 / 76.3 against 84.6 / 80.6 us.
// Measurement overrides: BSFP4_W4A16_ROWS64=0 never, =1 for any 5..128 rows.
bool w4a16_rows64_ok(int64_t M, int64_t N, int64_t K) {
  const char* e = getenv("BSFP4_W4A16_ROWS64");
  if (e && e[0] == '0') return false;
  const bool force = e && e[0] == '1';
  const int64_t min_rows = force ? 5 : 17, max_rows = force ? kRMaxRows : kRW4A16Rows;
  const int64_t lim = (int64_t)1 << 31;
  return M >= min_rows && M <= max_rows && K % kRSK == 0 && M * K * 2 < lim && N * (K / 2) < lim &&
         rows64_splits(M, N, K, device_cu_count()) > 0;
}

size_t w4a16_rows64_workspace(int64_t M, int64_t N, int64_t K) {
  const int s = rows64_splits(M, N, K, device_cu_count());
  return s > 1 ? (size_t)s * M * N * sizeof(float) : 0;
}

// NVFP4 activations: used for 24..128 rows.  Measured cold at N = 4096,
// K = 7168 (both kernels, events) against the split / per-wave small-M
// kernels: M = 17 18.8 / 18.4 us, M = 32 19.8 / 20.2, M = 64 22.2 / 23.6;
// against the tiled kernel: M = 65 / 96 / 128 26.4 / 27.9 / 29.1 against
// 27.0 / 29.4 / 30.9 us.
// Measurement overrides: BSFP4_NVFP4_ROWS64=0 never, =1 for any 5..128 rows.
bool nvfp4_rows64_ok(int64_t M, int64_t N, int64_t K) {
  const char* e = getenv("BSFP4_NVFP4_ROWS64");
  if (e && e[0] == '0') return false;
  const bool force = e && e[0] == '1';
  const int64_t min_rows = force ? 5 : 24, max_rows = force ? kRMaxRows : kRNvfp4Rows;
  const int64_t lim = (int64_t)1 << 31;
  return M >= min_rows && M <= max_rows && K % kRSK == 0 && M * (K / 2) < lim && N * (K / 2) < lim &&
         rows64_splits(M, N, K, device_cu_count()) > 0;
}

namespace {
template <int AKIND>
hipError_t launch_rows64(const void* A, const uint8_t* SFA, const uint8_t* B, const uint8_t* SFB,
                         const float* alpha, uint16_t* D, int64_t M, int64_t N, int64_t K, float* part,
                         size_t part_bytes, hipStream_t stream) {
  const int splits = rows64_splits(M, N, K, device_cu_count());
  if (splits < 1 || (splits > 1 && (part == nullptr || part_bytes < (size_t)splits * M * N * sizeof(float))))
    return hipErrorInvalidValue;
  const unsigned grid = (unsigned)(((N + kRBN - 1) / kRBN) * splits);
  if (M <= 64)
    rows64_gemm<AKIND, 64><<<grid, kRNT, 0, stream>>>(A, SFA, B, SFB, alpha, D, (int)M, (int)N, (int)K, splits, part);
  else
    rows64_gemm<AKIND, 128><<<grid, kRNT, 0, stream>>>(A, SFA, B, SFB, alpha, D, (int)M, (int)N, (int)K, splits, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  return launch_splitk_reduce(part, splits, alpha, D, M * N, stream);
}
}  // namespace

hipError_t launch_w4a16_rows64(const uint16_t* A, const uint8_t* B, const uint8_t* SFB, const float* alpha,
                               uint16_t* D, int64_t M, int64_t N, int64_t K, float* part, size_t part_bytes,
                               hipStream_t stream) {
  return launch_rows64<1>(A, nullptr, B, SFB, alpha, D, M, N, K, part, part_bytes, stream);
}

hipError_t launch_nvfp4_rows64(const uint8_t* A, const uint8_t* SFA, const uint8_t* B, const uint8_t* SFB,
                               const float* alpha, uint16_t* D, int64_t M, int64_t N, int64_t K, float* part,
                               size_t part_bytes, hipStream_t stream) {
  return launch_rows64<0>(A, SFA, B, SFB, alpha, D, M, N, K, part, part_bytes, stream);
}

}  // namespace bsfp4

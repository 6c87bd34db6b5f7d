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
// Structure (one workgroup = 256 threads = 4 waves in a 2x2 grid):
//   * BM x BN output tile, K walked in stages of 128 elements (64 code bytes and
//     8 scale bytes per row);
//   * each stage's packed codes and scale bytes are loaded from HBM with 128-bit
//     loads into registers one stage ahead, then stored to LDS (double buffered)
//     in a chunk-swizzled layout that keeps the MFMA fragment reads free of bank
//     conflicts;
//   * every wave reads its fragments from LDS as packed FP4 (4x less LDS traffic
//     than fp16 tiles), dequantises them in registers and issues
//     v_mfma_f32_32x32x16_f16 on a (BM/2) x (BN/2) wave tile;
//   * epilogue: alpha * acc, RNE to bf16, bounds-checked stores.
//
// MFMA lane layouts (measured on gfx950): for 32x32x16, lane l supplies row
// l%32 and eight consecutive K values of group l/32 of each operand; output
// register r of lane l holds row 8*(r/4) + 4*(l/32) + r%4, column l%32.  Within
// a stage the K index assigned to a lane's values is a fixed permutation shared
// by A and B, which leaves the sum unchanged; each lane's eight values always
// lie inside one 16-element scale block.
#include <algorithm>
#include <cstdlib>
#include <cstring>

#include "device_common.h"
#include "launchers.h"
#include "quant_device.h"

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

// Two E4M3 scale bytes (low 16 bits of `pair`) -> packed fp16 pair, exact.
// Placing the 7 magnitude bits of an E4M3 code at fp16 bit 7 gives the E4M3
// value times 2^-8 for normal and subnormal codes alike; one multiply by 256
// (exact) restores it.
__device__ __forceinline__ v2h e4m3x2_to_f16x2(uint32_t pair) {
  const uint32_t bits = ((pair & 0x7Fu) << 7) | ((pair & 0x7F00u) << 15);
  v2h h = __builtin_bit_cast(v2h, bits);
  const v2h k256 = {(_Float16)256.0f, (_Float16)256.0f};
  return h * k256;
}

// Eight E2M1 values (one 32-bit word, first value in the low nibble) times the
// fp16 scale `s` -> eight fp16 values, exact.
__device__ __forceinline__ v8h dequant8(uint32_t word, _Float16 s) {
  const v2h ss = {s, s};
  const v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 0) * ss;
  const v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 1) * ss;
  const v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 2) * ss;
  const v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 3) * ss;
  const v4h lo = __builtin_shufflevector(p0, p1, 0, 1, 2, 3);
  const v4h hi = __builtin_shufflevector(p2, p3, 0, 1, 2, 3);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
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

// ---------------------------------------------------------------------------
// Dequantise-once variant.  Each workgroup converts every E2M1 value of its
// tile exactly once, while writing a K stage into LDS, and the waves then read
// ready fp16 fragments (each fragment is read by two or four waves, which with
// per-wave dequantisation costs ~9 VALU instructions per MFMA; here ~2).
//
// Memory side.  Codes and scales are fetched in groups of 128 K values (two
// LDS stages) with buffer loads: four consecutive lanes read the four 16-byte
// chunks of one row's 64 bytes, so every load instruction touches 16 cache
// lines instead of 32, and the scale bytes of those chunks come from one line
// per row.  Rows outside the matrix and K beyond the tile's range read as zero
// (buffer range check, no branches).  Lane m of a quad takes chunk
// 2*((i + m/2) % 2) + m%2 in its i-th load, so each lane holds chunks of both
// LDS stages of the group and the dequantisation work is balanced.
//
// Pipeline.  A group's registers hold two LDS stages.  While the waves run the
// MFMAs of stage s from LDS slot s%2 they dequantise stage s+1 into the other
// slot (word by word between the MFMAs); one barrier per stage.  The next
// group is loaded at the top of the current one, a full stage before its
// first use.
// LDS: two fp16 stages, rows of 64 values padded to 144 B, so 16 lanes reading
// the same 16-byte chunk of 16 consecutive rows hit distinct bank groups and
// every fragment address is a per-lane base plus a constant; see f16_row for
// the write side.
// The MFMA takes the B fragment as its first operand, so each lane ends with
// four consecutive output columns of one row: the epilogue scales by alpha,
// rounds to bf16 and writes 8-byte vectors (FP32 16-byte vectors for split-K
// partials).
constexpr int kF16StageK = 64;   // K values per fp16 LDS stage
constexpr int kGroupK = 128;     // K values per load group
constexpr int kF16Pitch = 144;   // LDS bytes per row of a stage (128 + 16 padding)
constexpr uint32_t kOOB = 0x80000000u;  // buffer offset past every operand: loads return 0

// LDS byte offset of row R (A rows 0..BM-1, then B rows) in an fp16 stage of
// a workgroup of NT threads.  128-bit LDS writes are served 8 lanes (128 B,
// 32 banks) at a time: a quad writes 16-byte units of rows R and R + NT/4, the
// next quad those of R+1 and R+1+NT/4.  Shifting alternate NT/4-row blocks by
// 32 B puts the 8 units of such a lane group in distinct 32-bank positions
// (the 144-byte pitch moves each row by one unit).  The shift boundaries are
// multiples of 32 rows, so a 32-row fragment block never straddles one.
template <int NT>
__device__ __forceinline__ constexpr int f16_row(int R) {
  return R * kF16Pitch + ((R + NT / 4) / (NT / 2)) * 32;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// The thread's chunks of one load group: chunk i is row (tid + i*NT)/4 of the
// workgroup's BM + BN rows (A rows first).
template <int BM, int BN, int NT>
struct Fp4Group {
  static constexpr int kChunks = (BM + BN) * 4 / NT;
  static_assert((BM * 4) % NT == 0 && kChunks % 2 == 0, "operand split per load");
  uint4 code[kChunks];
  uint32_t sc[kChunks];  // the chunk's two E4M3 scale bytes
};

// Per-lane part of the buffer offsets; load i adds i*NT/4 rows (uniform) and
// its chunk's column.  Rows outside the matrix get kOOB.
template <int BM, int BN, int NT>
struct Fp4GroupOffsets {
  int64_t K;
  int r0, m, mrows, nrows;  // lane's row in load 0, lane in quad, valid A / B rows of the tile
  __device__ __forceinline__ Fp4GroupOffsets(int m0, int M, int n0, int N, int64_t K_, int tid)
      : K(K_), r0(tid >> 2), m(tid & 3), mrows(M - m0), nrows(N - n0) {}
  __device__ __forceinline__ int chunk(int i) const { return (i & 1) ? (m ^ 2) : m; }
};

template <int BM, int BN, int NT>
__device__ __forceinline__ void fp4_group_load(Fp4Group<BM, BN, NT>& g, __amdgpu_buffer_rsrc_t ra_q,
                                               __amdgpu_buffer_rsrc_t ra_s, __amdgpu_buffer_rsrc_t rb_q,
                                               __amdgpu_buffer_rsrc_t rb_s, const Fp4GroupOffsets<BM, BN, NT>& o,
                                               int64_t k0, int64_t k_end) {
  constexpr int kA = BM * 4 / NT;  // loads of A rows
#pragma unroll
  for (int i = 0; i < Fp4Group<BM, BN, NT>::kChunks; i++) {
    const bool is_a = i < kA;
    const int r = o.r0 + (is_a ? i : i - kA) * (NT / 4);  // row inside the operand's tile rows
    const int c = o.chunk(i);
    const bool live = r < (is_a ? o.mrows : o.nrows) && k0 + c * 32 < k_end;
    // offsets are relative to the tile's first row (the buffer base)
    const uint32_t oc = live ? (uint32_t)(r * (o.K / 2) + c * 16 + k0 / 2) : kOOB;
    const uint32_t os = live ? (uint32_t)(r * (o.K / 16) + c * 2 + k0 / 16) : kOOB;
    g.code[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(is_a ? ra_q : rb_q, (int)oc, 0, 0));
    g.sc[i] = __builtin_amdgcn_raw_buffer_load_b16(is_a ? ra_s : rb_s, (int)os, 0, 0);
  }
}

// Word W of the thread's stage-H share of group g -> 8 fp16 values in LDS stage
// `lds`.  The share is chunk pair j = W/4: load 2j or 2j+1, whichever holds
// stage H for this lane.
template <int W, int H, int BM, int BN, int NT>
__device__ __forceinline__ void group_word_store(const Fp4Group<BM, BN, NT>& g, uint8_t* lds, int tid) {
  constexpr int j = W / 4, w = W % 4;
  const int m = tid & 3;
  const bool odd = ((m >> 1) ^ H) & 1;  // this lane's stage-H chunk is load 2j+1
  const uint4 c0 = g.code[2 * j], c1 = g.code[2 * j + 1];
  const uint32_t word = w == 0 ? (odd ? c1.x : c0.x)
                      : w == 1 ? (odd ? c1.y : c0.y)
                      : w == 2 ? (odd ? c1.z : c0.z)
                               : (odd ? c1.w : c0.w);
  const uint32_t scp = odd ? g.sc[2 * j + 1] : g.sc[2 * j];
  const v2h s01 = e4m3x2_to_f16x2(scp);  // words 0,1 take scale 0; words 2,3 scale 1
  // row of load 2j (+NT/4 rows for load 2j+1); position of the chunk in the stage row
  const int r = ((tid + 2 * j * NT) >> 2) + (odd ? NT / 4 : 0);
  *reinterpret_cast<v8h*>(lds + f16_row<NT>(r) + ((m & 1) * 4 + w) * 16) = dequant8(word, w < 2 ? s01.x : s01.y);
}

// qa / qb: the stage slot plus the lane's row and K-half offset; fragment i of
// A is row block wm*WM + 32i, fragment j of B row block BM + wn*WN + 32j.
template <int BM, int BN, int WGM, int WGN>
__device__ __forceinline__ void f16_stage_compute(const uint8_t* qa, const uint8_t* qb,
                                                  v16f (&acc)[BM / WGM / 32][BN / WGN / 32],
                                                  const Fp4Group<BM, BN, 64 * WGM * WGN>& g, uint8_t* nx, int tid,
                                                  bool store_h1, int wm, int wn) {
  // store_h1: dequantise this group's stage 1 (else the next group's stage 0,
  // which the caller passes as g)
  constexpr int NT = 64 * WGM * WGN;
  constexpr int TM = BM / WGM / 32, TN = BN / WGN / 32;
  constexpr int kWords = 4 * Fp4Group<BM, BN, NT>::kChunks / 2;  // words of one stage per thread
  constexpr int kWordsPerStep = kWords / 4;
  constexpr int kMfma = TM * TN;
  static_assert(kWordsPerStep >= 1 && kWordsPerStep <= kMfma, "word spread");
  // The dequantisation of the next stage is spread word by word between the
  // MFMAs; scheduling fences keep this order (the compiler would otherwise
  // hoist all LDS reads and VALU work above the MFMAs).
#pragma unroll
  for (int kk = 0; kk < kF16StageK / 16; kk++) {
    v8h fa[TM], fb[TN];
#pragma unroll
    for (int j = 0; j < TN; j++)
      fb[j] = *reinterpret_cast<const v8h*>(qb + f16_row<NT>(BM + wn * (BN / WGN) + j * 32) + kk * 32);
#pragma unroll
    for (int i = 0; i < TM; i++)
      fa[i] = *reinterpret_cast<const v8h*>(qa + f16_row<NT>(wm * (BM / WGM) + i * 32) + kk * 32);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < kMfma; t++) {
      const int i = t / TN, j = t % TN;
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fb[j], fa[i], acc[i][j], 0, 0, 0);
#pragma unroll
      for (int w = 0; w < kWordsPerStep; w++) {
        if (t == (w * kMfma) / kWordsPerStep) {
          switch (kk * kWordsPerStep + w) {  // compile-time after unrolling
#define BSFP4_W(x)                                                              \
  case x:                                                                       \
    if constexpr (x < kWords) {                                                 \
      if (store_h1)                                                             \
        group_word_store<x, 1, BM, BN, NT>(g, nx, tid);                         \
      else                                                                      \
        group_word_store<x, 0, BM, BN, NT>(g, nx, tid);                         \
    }                                                                           \
    break;
            BSFP4_W(0) BSFP4_W(1) BSFP4_W(2) BSFP4_W(3) BSFP4_W(4) BSFP4_W(5) BSFP4_W(6) BSFP4_W(7)
            BSFP4_W(8) BSFP4_W(9) BSFP4_W(10) BSFP4_W(11) BSFP4_W(12) BSFP4_W(13) BSFP4_W(14) BSFP4_W(15)
#undef BSFP4_W
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

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

// ---------------------------------------------------------------------------
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

int device_cus() {
  static int n = 0;
  if (n == 0) {
    int dev = 0, v = 0;
    n = (hipGetDevice(&dev) == hipSuccess &&
         hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
            ? v
            : 256;
  }
  return n;
}

}  // namespace

// 256x256 tiles: the dequantise-once kernel with 8 waves of 128x64 by default.
// BSFP4_NVFP4_KERNEL selects an alternative for measurements: "lds4" (same
// kernel, 4 waves of 128x128), "reg8" / "reg4" (per-wave register
// dequantisation, 8 or 4 waves).
// The dequantise-once kernel addresses operands with 32-bit buffer offsets
// (M*K/2 and N*K/2 below 2^31); larger operands take the register-dequant
// kernel.
static int nvfp4_variant(int64_t M, int64_t N, int64_t K) {
  const char* e = getenv("BSFP4_NVFP4_KERNEL");
  int v = 0;
  if (e && !strcmp(e, "lds4")) v = 1;
  if (e && !strcmp(e, "reg8")) v = 2;
  if (e && !strcmp(e, "reg4")) v = 3;
  const int64_t lim = (int64_t)1 << 31;
  if ((v == 0 || v == 1) && (M * (K / 2) >= lim || N * (K / 2) >= lim)) v = 2;
  return v;
}

hipError_t launch_nvfp4_gemm(const uint8_t* A, const uint8_t* SFA, const uint8_t* B, const uint8_t* SFB,
                             const float* alpha, uint16_t* D, int64_t M, int64_t N, int64_t K,
                             void* ws, size_t ws_bytes, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  if (M <= kSkinnyMaxM)
    return launch_skinny_nvfp4(A, SFA, B, SFB, alpha, D, M, N, K, static_cast<float*>(ws), stream);
  const int v = nvfp4_variant(M, N, K);
  Plan pl = plan_tiled(M, N, K, device_cus(), v < 2);
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
      default: nvfp4_gemm_f16lds<256, 256, 2, 4><<<grid, 512, 0, stream>>>(BSFP4_ARGS, tiles_m, tiles_n, pl.splits, part);
    }
  } else if (pl.bm == 256) {  // 256x128 (planned only for the dequantise-once kernels)
    nvfp4_gemm_f16lds<256, 128, 2, 2><<<grid, 256, 0, stream>>>(BSFP4_ARGS, tiles_m, tiles_n, pl.splits, part);
  } else {
    if (v >= 2)
      nvfp4_gemm_tiled<128, 128, 2, 2><<<grid, 256, 0, stream>>>(BSFP4_ARGS, tiles_n, pl.splits, part);
    else
      nvfp4_gemm_f16lds<128, 128, 2, 2><<<grid, 256, 0, stream>>>(BSFP4_ARGS, tiles_m, tiles_n, pl.splits, part);
  }
#undef BSFP4_ARGS
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.splits == 1) return e;
  const int64_t q = M * N / 4;
  const unsigned rgrid = (unsigned)((q + 255) / 256 > 16384 ? 16384 : (q + 255) / 256);
  splitk_reduce<<<rgrid, 256, 0, stream>>>(part, pl.splits, alpha, D, M * N);
  return hipGetLastError();
}

hipError_t launch_splitk_reduce(const float* part, int splits, const float* alpha, uint16_t* D, int64_t MN,
                                hipStream_t stream) {
  const int64_t q = MN / 4;
  const unsigned rgrid = (unsigned)((q + 255) / 256 > 16384 ? 16384 : (q + 255) / 256);
  splitk_reduce<<<rgrid < 1 ? 1 : rgrid, 256, 0, stream>>>(part, splits, alpha, D, MN);
  return hipGetLastError();
}

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
  int64_t grid = 2 * (int64_t)device_cus();
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

size_t nvfp4_gemm_workspace(int64_t M, int64_t N, int64_t K) {
  if (M <= kSkinnyMaxM) return skinny_workspace(M, N, K, true);
  const Plan pl = plan_tiled(M, N, K, device_cus(), nvfp4_variant(M, N, K) < 2);
  return pl.splits > 1 ? (size_t)pl.splits * M * N * sizeof(float) : 0;
}

}  // namespace bsfp4

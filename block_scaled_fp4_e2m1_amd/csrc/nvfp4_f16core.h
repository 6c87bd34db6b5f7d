// The exact NVFP4 dequantise-to-fp16 GEMM core shared by the dense
// (gemm_nvfp4.hip) and the grouped-by-expert (moe_nvfp4.hip) kernels:
// E4M3 scale and E2M1 value conversions to fp16, the load groups of packed
// codes and scales, their dequantisation into LDS and the MFMA stage loop.
#pragma once

#include "device_common.h"

namespace bsfp4 {
namespace {

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


}  // namespace
}  // namespace bsfp4

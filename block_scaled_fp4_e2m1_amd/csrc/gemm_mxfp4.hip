// MXFP4 W4A4 GEMM on gfx950's scaled FP4 MFMA, dense and grouped by expert.
//
//   dense:    D[m, n]  = bf16(alpha * sum_k dec(A)[m,k] * dec(B)[n,k])
//   grouped:  rows [off[e], off[e+1]) of A times expert e's weights W[e]
//
// The MXFP4 form of the block-scaled GEMM (E2M1 values, one E8M0 scale per 32
// K-elements) and the MXFP4 x MXFP4 per-expert grouped GEMM of "[Kernel]
// Enable CUTLASS MXFP4 W4A4 MoE on SM12x".  Its scales are exactly what
// v_mfma_scale_f32_32x32x64_f8f6f4 applies: lane l supplies 32 E2M1 values of
// row l%32 (K group l/32) in 16 bytes plus that block's E8M0 byte, so the
// packed codes and scale bytes go from HBM to the matrix cores untouched.
//
// Workgroups of 2 x WGN waves own a BM x BN tile (dense: 256 x 256, 8 waves;
// grouped: 128 x 128, 4 waves).  K runs in stages of SK values (SK/2 code bytes
// + SK/32 scale bytes per row) through an LDS ring filled by direct-to-LDS
// buffer loads (256-value stages, whole 128-byte rows per request, when
// K % 256 == 0; else 128-value stages), with a 16-byte-chunk swizzle that keeps
// the fragment reads conflict-free; shapes with K % 128 != 0 use a
// register-staged double buffer.  The grid is persistent: each workgroup walks
// a list of (group, column tile, row tile) work items with row tiles innermost;
// consecutive items are assigned to workgroups of the same XCD so that row tiles
// that share a weight panel run on one L2.  The item list is built in LDS from
// the per-expert offsets at kernel start: a group with m rows contributes
// ceil(m / BM) * ceil(N / BN) items, so the load follows the routing.
//
// Epilogues:
//   STORE    alpha * acc -> bf16 rows;
//   SILU     the tile's columns are gate/up pairs: column blocks of 32 alternate
//            gate rows [32b, 32b+32) and up rows [N/2 + 32b, ...) of W, so a lane
//            holds gate and up of the same element; act = bf16(silu(h_g) * h_u)
//            from the bf16-rounded h (SiLU with the hardware exp2 and reciprocal),
//            staged in LDS and re-quantised to MXFP4 per 32-element block with
//            the hardware bf16 -> E2M1 conversion (the fused
//            `silu_and_mul_scaled_fp4_experts_quant` pattern of the vLLM `sm103`
//            branch comparison page, MXFP4 form);
//   COMBINE  y[f] = row in FP32 for the row's flat (token, slot) index f; a
//            second kernel sums topk_weight[f] * y[f] over each token's slots in
//            slot order and rounds once to bf16 (deterministic; the same layer
//            with device-wide float atomics for the combine measured about 2x
//            slower).  The tile's f indices are loaded when the tile starts and
//            reach the epilogue through LDS.
#include <cstdlib>
#include <cstring>

#include "device_common.h"
#include "launchers.h"
#include "lds_dma.h"
#include "quant_device.h"

namespace bsfp4 {
namespace {


// Stage geometry for SK K-values per stage: SK/2 code bytes (SK/32 chunks of 16
// bytes) and SK/32 E8M0 bytes per row.
template <int SK>
struct Geo {
  static constexpr int kRowBytes = SK / 2;
  static constexpr int kChunks = SK / 32;   // 16-byte chunks per row
  static constexpr int kRowScales = SK / 32;
  // chunk position inside the row: 8 (or 16) lanes reading the same logical
  // chunk of 8 (or 16) consecutive rows hit distinct 16-byte bank groups
  __device__ static __forceinline__ int swz(int r, int c) {
    if constexpr (kChunks == 8) return c ^ ((r ^ (r >> 3)) & 7);
    else return c ^ (((r >> 1) ^ (r >> 3)) & 3);
  }
};

template <int ROWS, int SK, int NT>
struct Stage {
  static constexpr int kChunks = ROWS * Geo<SK>::kChunks / NT;
  uint4 code[kChunks];
  uint32_t sc[Geo<SK>::kRowScales / 4];
};

// Loads one stage of ROWS rows.  Row i of the tile is global row rowmap(i);
// rows at or beyond `nvalid` (and rowmap < 0) read as zero.
template <int ROWS, int SK, int NT, class RowMap>
__device__ __forceinline__ void load_stage(Stage<ROWS, SK, NT>& st, const uint8_t* __restrict__ q,
                                           const uint8_t* __restrict__ sf, RowMap rowmap, int nvalid,
                                           int K, int k0, bool sc_aligned, int tid) {
  using Gm = Geo<SK>;
  const int row_bytes = K / 2, row_blocks = K / 32;
#pragma unroll
  for (int i = 0; i < Stage<ROWS, SK, NT>::kChunks; i++) {
    const int idx = tid + i * NT;
    const int r = idx / Gm::kChunks, c = idx % Gm::kChunks;
    const int gr = rowmap(r);
    const int kb = k0 / 2 + c * 16;
    st.code[i] = (gr >= 0 && gr < nvalid && kb < row_bytes)
                     ? *reinterpret_cast<const uint4*>(q + (int64_t)gr * row_bytes + kb)
                     : make_uint4(0, 0, 0, 0);
  }
  if (tid < ROWS) {
    constexpr int kW = Gm::kRowScales / 4;  // scale words per row per stage
    const int gr = rowmap(tid);
#pragma unroll
    for (int j = 0; j < kW; j++) st.sc[j] = 0;
    if (gr >= 0 && gr < nvalid) {
      const int b0 = k0 / 32;
      const uint8_t* p = sf + (int64_t)gr * row_blocks;
      if (sc_aligned && b0 + Gm::kRowScales <= row_blocks) {
        if constexpr (kW == 2) {
          const uint2 v = *reinterpret_cast<const uint2*>(p + b0);
          st.sc[0] = v.x;
          st.sc[1] = v.y;
        } else {
          st.sc[0] = *reinterpret_cast<const uint32_t*>(p + b0);
        }
      } else {
#pragma unroll
        for (int j = 0; j < Gm::kRowScales; j++) {
          const uint32_t b = (b0 + j < row_blocks) ? p[b0 + j] : 0u;
          st.sc[j / 4] |= b << (8 * (j % 4));
        }
      }
    }
  }
}

template <int ROWS, int SK, int NT>
__device__ __forceinline__ void store_stage(const Stage<ROWS, SK, NT>& st, uint8_t* lq, uint8_t* ls, int tid) {
  using Gm = Geo<SK>;
#pragma unroll
  for (int i = 0; i < Stage<ROWS, SK, NT>::kChunks; i++) {
    const int idx = tid + i * NT;
    const int r = idx / Gm::kChunks, c = idx % Gm::kChunks;
    *reinterpret_cast<uint4*>(lq + r * Gm::kRowBytes + Gm::swz(r, c) * 16) = st.code[i];
  }
  if (tid < ROWS) {
    if constexpr (Gm::kRowScales == 8)
      *reinterpret_cast<uint2*>(ls + tid * 8) = make_uint2(st.sc[0], st.sc[1]);
    else
      *reinterpret_cast<uint32_t*>(ls + tid * 4) = st.sc[0];
  }
}

struct Args {
  const uint8_t* A;
  const uint8_t* SFA;
  int rows;
  const int32_t* a_rows;   // optional: row m of the problem reads row a_rows[m] of A
  int a_nrows;             // rows of A (bounds of a_rows entries)
  const int32_t* offsets;  // nullptr: one group holding every row
  int E;
  const uint8_t* W;
  const uint8_t* WSF;
  int N;
  int K;
  const float* alpha;
  uint16_t* out;           // STORE: bf16 [rows, N]
  uint8_t* out_q;          // SILU: [rows, N/4]
  uint8_t* out_sf;         // SILU: [rows, N/64]
  const int32_t* sorted_ids;  // COMBINE
  float* y_f32;               // COMBINE: [T * topk, N], row f = flat (token, slot) index
};

constexpr int kMaxGroups = (int)kMaxExperts;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Workgroups per CU the register budget is sized for: small tiles keep two
// resident so that one's loads overlap the other's MFMAs.
// kDMA: an RING-stage LDS ring filled by direct-to-LDS buffer loads, stages of
// SK = 128 values (64 code bytes per row: each load moves 16 rows x 64 B;
// K % 128 == 0) or SK = 256 values (128 B per row: each load moves 8 rows x
// 128 B, whole cache lines, which the memory pipeline serves at a higher rate
// per request; K % 256 == 0).  Otherwise: register-staged double buffer, any
// K % 32.
// The two-slot ring of 256-value stages takes its E8M0 scales in chunks of two
// stages (16 bytes per row), double-buffered beside the code slots: one
// 16-byte lane per row when a row's scale bytes are 16-byte aligned (K % 512
// == 0; one load per wave and chunk for the 256 x 256 and 128 x 128 tiles),
// else four 4-byte lanes per row (16 rows per load instead of the 32 of
// per-stage loads).  Measured on the dense 4096 x 4096 x 7168 GEMM, cold:
// 81.4 us with per-stage scale loads, 76.8 with 4-byte-lane chunks, 74.1
// with 16-byte-lane chunks (without any scale loads, a timing-only variant:
// 65.4).  The other forms keep each stage's scales in its slot.
template <int SK, int RING>
constexpr bool chunked_scales() { return SK == 256 && RING == 2; }
constexpr int kScChunkRow = 16;  // scale bytes of one row in a chunk (2 stages x 8)

template <int BM, int BN, int SK, int RING>
constexpr int ring_lds_bytes() {
  return chunked_scales<SK, RING>() ? RING * (BM + BN) * (SK / 2) + 2 * (BM + BN) * kScChunkRow
                                    : RING * (BM + BN) * (SK / 2 + SK / 32);
}

// Workgroups per CU the register budget and LDS are sized for: small tiles keep
// two resident so that one's loads overlap the other's MFMAs (when two rings fit
// in the 160 KB of LDS).
template <int BM, int BN, int SK, int RING>
constexpr int wg_per_cu() {
  return (BM * BN <= 128 * 128 && 2 * (ring_lds_bytes<BM, BN, SK, RING>() + 2048) <= 160 * 1024) ? 2 : 1;
}

// kLoaders: waves that issue the ring's loads (0: all).
// SC16: the scale chunks move in 16-byte lanes (K % 512 == 0)
template <int BM, int BN, int WGN, int SK, int EPI, bool kDMA, int kLoaders, int RING, bool SC16 = false>
__global__ void __launch_bounds__(128 * WGN, (wg_per_cu<BM, BN, SK, RING>())) mxfp4_grouped(Args p) {
  constexpr int NT = 128 * WGN;  // 2 x WGN waves
  static_assert(!kDMA || SK == 128 || SK == 256, "the LDS ring uses 128- or 256-value stages");
  static_assert(!kDMA || (RING >= 2 && RING <= 4), "ring depth");
  using Gm = Geo<SK>;
  constexpr int kRowBytes = Gm::kRowBytes, kRowScales = Gm::kRowScales;
  constexpr int WM = BM / 2, WN = BN / WGN;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int kA = BM * kRowBytes, kB = BN * kRowBytes;
  constexpr bool kChunkSc = kDMA && chunked_scales<SK, RING>();
  constexpr int kStage = kA + kB + (kChunkSc ? 0 : (BM + BN) * kRowScales);
  constexpr int kChunkBytes = kChunkSc ? 2 * (BM + BN) * kScChunkRow : 0;  // two scale chunks after the ring
  static_assert(EPI != kEpiSilu || TN % 2 == 0, "SILU needs gate/up column-tile pairs");
  // With the B fragment as the MFMA's first operand a lane's accumulators run
  // along a row (4 consecutive columns per register quad).  SILU needs that
  // (the act block of a row sits in two lanes), and so does the LDS-staged
  // output of the ring kernel (8- or 16-byte LDS writes).  The register-staged
  // kernel stores STORE / COMBINE tiles directly and keeps A first: a lane
  // holds one column of 16 rows and each store writes 128 contiguous bytes.
  constexpr bool kSwap = EPI == kEpiSilu || kDMA;
  // LDS-staged output tile (ring kernel): bf16 or FP32 rows padded by 16 bytes
  constexpr int kOutElem = EPI == kEpiCombine ? 4 : 2;
  constexpr int kOutPitch = BN * kOutElem + 16;
  static_assert(!kDMA || EPI == kEpiSilu || BM * kOutPitch <= RING * kStage + kChunkBytes,
                "output tile fits in the ring");
  constexpr int kSlots = kDMA ? RING : 2;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kSlots * kStage + kChunkBytes];
  __shared__ int tile_start[kMaxGroups + 1];
  __shared__ int row_f[EPI == kEpiCombine ? BM : 1];
  __shared__ int wave_sum[NT / 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;
  const int lr = lane & 31, g = lane >> 5;
  const int ntn = (p.N + BN - 1) / BN;
  const int K = p.K;
  const bool sc_aligned = ((K / 32) % kRowScales) == 0;

  // ---- work list: tile_start[e] = items of groups before e
  int total;
  if (p.offsets == nullptr) {
    total = ((p.rows + BM - 1) / BM) * ntn;
  } else {
    // each thread owns up to 4 consecutive groups; block-wide exclusive scan
    int cnt[4];
    int local = 0;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int e = tid * 4 + j;
      int c = 0;
      if (e < p.E) {
        const int m = p.offsets[e + 1] - p.offsets[e];
        c = ((m + BM - 1) / BM) * ntn;
      }
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
    if (tid == NT - 1) tile_start[p.E] = base;  // the last thread owns the last groups
    __syncthreads();
    total = tile_start[p.E];
  }

  const int G = gridDim.x;
  const int slot = (G % 8 == 0) ? (int)(blockIdx.x % 8) * (G / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;
  const float alpha = p.alpha ? p.alpha[0] : 1.0f;

  for (int t = slot; t < total; t += G) {
    // ---- locate the work item
    int e = 0, row0, row_end, nmt;
    if (p.offsets == nullptr) {
      nmt = (p.rows + BM - 1) / BM;
      row0 = 0;
      row_end = p.rows;
    } else {
      int lo = 0, hi = p.E - 1;  // largest e with tile_start[e] <= t
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (tile_start[mid] <= t) lo = mid; else hi = mid - 1;
      }
      e = lo;
      row0 = p.offsets[e];
      row_end = p.offsets[e + 1];
      nmt = (row_end - row0 + BM - 1) / BM;
    }
    const int local = t - (p.offsets ? tile_start[e] : 0);
    int tn, tmi;
    if (p.offsets == nullptr) {
      // dense: bands of 4 row tiles, so that the 32 consecutive items an XCD
      // receives form a 4 x 8 block of tiles (fewer A and B panels per L2)
      const int band_items = 4 * ntn;
      const int band = local / band_items, in_band = local % band_items;
      const int band_rows = min(4, nmt - band * 4);
      tmi = band * 4 + in_band % band_rows;
      tn = in_band / band_rows;
    } else {
      tn = local / nmt;
      tmi = local % nmt;
    }
    const int m0 = row0 + tmi * BM;
    const int nvalid_a = row_end < p.rows ? row_end : p.rows;
    const uint8_t* Wq = p.W + (int64_t)e * p.N * (K / 2);
    const uint8_t* Ws = p.WSF + (int64_t)e * p.N * (K / 32);

    // A row of problem row m0 + i (-1: beyond this group / the problem)
    auto amap = [&](int i) -> int {
      const int m = m0 + i;
      if (m >= nvalid_a) return -1;
      return p.a_rows ? p.a_rows[m] : m;
    };
    const int a_lim = p.a_rows ? p.a_nrows : nvalid_a;
    auto bmap = [&](int i) -> int {
      if constexpr (EPI == kEpiSilu) {
        // LDS row i: wave column half wc = i / WN, column tile jn = (i % WN) / 32;
        // even jn = gate, odd jn = up, act block b = tn*(BN/64) + wc*(TN/2) + jn/2
        const int wc = i / WN, jn = (i % WN) >> 5;
        const int b = tn * (BN / 64) + wc * (TN / 2) + (jn >> 1);
        if (32 * b >= p.N / 2) return -1;
        return ((jn & 1) ? p.N / 2 : 0) + 32 * b + (i & 31);
      } else {
        return tn * BN + i;
      }
    };

    // COMBINE: flat index of tile row tid, loaded before the K loop's loads so
    // that it has arrived when the epilogue needs it
    int rf = -1;
    if constexpr (EPI == kEpiCombine) {
      if (tid < BM && m0 + tid < nvalid_a) rf = p.sorted_ids[m0 + tid];
    }

    v16f acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
      for (int j = 0; j < TN; j++) acc[i][j] = v16f{};

    const int nst = (K + SK - 1) / SK;
    if constexpr (kDMA) {
      // Direct-to-LDS ring, filled by kLoad waves (all waves, or the first
      // kLoaders).  Per stage: (BM+BN)/kRowsLoad code loads of kRowsLoad rows x
      // kRowBytes (1 KB each) and (BM+BN)/kScRowsLoad scale loads of 4 B per
      // lane; each lane keeps one 32-bit offset per load (kBufOOB for rows
      // outside the problem), the stage's K offset goes in the SGPR offset.
      constexpr int kWaves = NT / 64;
      constexpr int kLoad = kLoaders > 0 ? kLoaders : kWaves;
      constexpr int kLanesRow = kRowBytes / 16;        // lanes per row of a code load
      constexpr int kRowsLoad = 64 / kLanesRow;         // rows per code load (16 or 8)
      constexpr int kScLanesRow = kRowScales / 4;       // lanes per row of a scale load
      constexpr int kScRowsLoad = 64 / kScLanesRow;     // rows per scale load (64 or 32)
      constexpr int kCodeI = (BM + BN) / kRowsLoad / kLoad;
      constexpr int kScaleI = (BM + BN) / kScRowsLoad / kLoad;
      static_assert(kCodeI * kLoad * kRowsLoad == BM + BN && kScaleI * kLoad * kScRowsLoad == BM + BN,
                    "DMA loads must cover the tile rows exactly");
      static_assert(BM % kScRowsLoad == 0 && BM % kRowsLoad == 0, "a load holds rows of one operand");
      constexpr int kL = kCodeI + kScaleI;  // ring loads per loading wave per stage
      const bool loader = wave < kLoad;
      const v4u32 ra_q = make_rsrc4(p.A, (int64_t)a_lim * (K / 2));
      const v4u32 ra_s = make_rsrc4(p.SFA, (int64_t)a_lim * (K / 32));
      const v4u32 rw_q = make_rsrc4(Wq, (int64_t)p.N * (K / 2));
      const v4u32 rw_s = make_rsrc4(Ws, (int64_t)p.N * (K / 32));
      uint32_t cv[kCodeI], sv[kScaleI];
#pragma unroll
      for (int j = 0; j < kCodeI; j++) {
        const int q = (loader ? wave : 0) * kCodeI + j;  // load index in the stage
        const bool isA = q < BM / kRowsLoad;
        const int qq = isA ? q : q - BM / kRowsLoad;
        const int row = qq * kRowsLoad + lane / kLanesRow;  // tile row of this lane's chunk
        const int c = Gm::swz(row, lane % kLanesRow);       // logical chunk landing at LDS position lane % kLanesRow
        const int gr = isA ? amap(row) : bmap(row);
        const bool ok = gr >= 0 && gr < (isA ? a_lim : p.N);
        cv[j] = ok ? (uint32_t)(gr * (K / 2) + c * 16) : kBufOOB;
      }
#pragma unroll
      for (int j = 0; j < kScaleI; j++) {
        const int q = (loader ? wave : 0) * kScaleI + j;
        const bool isA = q < BM / kScRowsLoad;
        const int qq = isA ? q : q - BM / kScRowsLoad;
        const int row = qq * kScRowsLoad + lane / kScLanesRow;
        const int gr = isA ? amap(row) : bmap(row);
        const bool ok = gr >= 0 && gr < (isA ? a_lim : p.N);
        sv[j] = ok ? (uint32_t)(gr * (K / 32) + (lane % kScLanesRow) * 4) : kBufOOB;
      }
      // chunked scales: load j of the wave covers kChRows tile rows (A rows,
      // then B rows) from row kChRows (kChI wave + j): 16-byte lanes, row
      // + lane; or 4-byte lanes, row + lane / 4, where dword d of a row's 16
      // chunk bytes lands at position d ^ ((row >> 3) & 3) so that 32 rows'
      // dword reads hit distinct banks
      constexpr int kChRows = SC16 ? 64 : 16;
      constexpr int kChI = kChunkSc ? (BM + BN) / kChRows / kWaves : 1;
      static_assert(!kChunkSc || (kChI * kChRows * kWaves == BM + BN && kLoad == kWaves && BM % kChRows == 0),
                    "scale chunk loads cover the tile rows, every wave loading");
      auto sc_pos = [](int row, int d) { return SC16 ? d : d ^ ((row >> 3) & 3); };
      uint32_t cv_sc[kChI];
#pragma unroll
      for (int j = 0; j < kChI; j++) {
        const int row = kChRows * (kChI * wave + j) + (SC16 ? lane : lane / 4);
        const bool isA = row < BM;
        const int gr = isA ? amap(row) : bmap(row - BM);
        const bool ok = kChunkSc && gr >= 0 && gr < (isA ? a_lim : p.N);
        cv_sc[j] = ok ? (uint32_t)(gr * (K / 32) + (SC16 ? 0 : sc_pos(row, lane & 3) * 4)) : kBufOOB;
      }
      const uint32_t lds0 = lds_offset(smem);
      uint8_t* const chunk0 = smem + RING * kStage;  // [chunk % 2][tile rows][16 B]
      auto issue = [&](int st) {
        const uint32_t slot = lds0 + (uint32_t)((st % RING) * kStage);
#pragma unroll
        for (int j = 0; j < kCodeI; j++) {
          const int q = wave * kCodeI + j;
          const bool isA = q < BM / kRowsLoad;
          const uint32_t dst = slot + (uint32_t)((isA ? 0 : kA) + (isA ? q : q - BM / kRowsLoad) * 1024);
          buf_lds16(uniform4(isA ? ra_q : rw_q), cv[j], (uint32_t)(st * (SK / 2)),
                    (uint32_t)__builtin_amdgcn_readfirstlane((int)dst));
        }
        if constexpr (kChunkSc) {
          if (st % 2 == 0) {  // the chunk of stages st, st + 1
            uint8_t* buf = chunk0 + ((st / 2) & 1) * ((BM + BN) * kScChunkRow);
#pragma unroll
            for (int j = 0; j < kChI; j++) {
              const bool isA = kChRows * (kChI * wave + j) < BM;
              const uint32_t dst =
                  (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_offset(buf + (kChI * wave + j) * kChRows * 16));
              if constexpr (SC16)
                buf_lds16(uniform4(isA ? ra_s : rw_s), cv_sc[j], (uint32_t)(st * (SK / 32)), dst);
              else
                buf_lds4(uniform4(isA ? ra_s : rw_s), cv_sc[j], (uint32_t)(st * (SK / 32)), dst);
            }
          }
        } else {
#pragma unroll
          for (int j = 0; j < kScaleI; j++) {
            const int q = wave * kScaleI + j;
            const bool isA = q < BM / kScRowsLoad;
            const uint32_t dst =
                slot + (uint32_t)(kA + kB + (isA ? 0 : BM * kRowScales) + (isA ? q : q - BM / kScRowsLoad) * 256);
            buf_lds4(uniform4(isA ? ra_s : rw_s), sv[j], (uint32_t)(st * (SK / 32)),
                     (uint32_t)__builtin_amdgcn_readfirstlane((int)dst));
          }
        }
      };
      if (loader)
        for (int st = 0; st < RING - 1 && st < nst; st++) issue(st);
      for (int s = 0; s < nst; s++) {
        if (loader) {
          const int ahead = min(RING - 2, nst - 1 - s);  // stages issued after s
          if (ahead >= 2) wait_vmcnt<2 * kL>();
          else if (ahead == 1) wait_vmcnt<kL>();
          else wait_vmcnt<0>();
        }
        __builtin_amdgcn_s_barrier();  // stage s visible; every wave is past stage s-1
        if (loader && s + RING - 1 < nst) issue(s + RING - 1);
        const uint8_t* st = smem + (s % RING) * kStage;
        const uint8_t* qa = st;
        const uint8_t* qb = st + kA;
        const uint8_t* sa = st + kA + kB;
        const uint8_t* sb = sa + BM * kRowScales;
        // the scale bytes of a fragment row, one dword per 4 (lanes g = 0 / 1
        // of a row read the same dwords), shifted so that byte 2(j%2) of dword
        // j/2 is this lane's chunk 2j + g; the MFMA's op_sel picks that byte
        constexpr int kScW = kRowScales / 4;
        const uint8_t* chs = chunk0 + ((s / 2) & 1) * ((BM + BN) * kScChunkRow);  // chunked: [tile row][16 B]
        auto sc_word = [&](int row, int d) {  // dword d of this stage's scale bytes of tile row `row`
          if constexpr (kChunkSc)
            return *reinterpret_cast<const uint32_t*>(chs + row * kScChunkRow + sc_pos(row, (s & 1) * kScW + d) * 4);
          else
            return *reinterpret_cast<const uint32_t*>(row < BM ? sa + row * kRowScales + 4 * d
                                                               : sb + (row - BM) * kRowScales + 4 * d);
        };
        uint32_t xa4[TM][kScW], xb4[TN][kScW];
#pragma unroll
        for (int i = 0; i < TN; i++)
#pragma unroll
          for (int d = 0; d < kScW; d++) xb4[i][d] = sc_word(BM + wn * WN + i * 32 + lr, d) >> (8 * g);
#pragma unroll
        for (int i = 0; i < TM; i++)
#pragma unroll
          for (int d = 0; d < kScW; d++) xa4[i][d] = sc_word(wm * WM + i * 32 + lr, d) >> (8 * g);
#pragma unroll
        for (int j = 0; j < SK / 64; j++) {
          const int c = 2 * j + g;  // 16-byte chunk = K values 64j + 32g .. +32 of the stage
          v8i fb[TN];
  #pragma unroll
          for (int i = 0; i < TN; i++) {
            const int r = wn * WN + i * 32 + lr;
            const uint4 v = *reinterpret_cast<const uint4*>(qb + r * kRowBytes + Gm::swz(r, c) * 16);
            fb[i] = v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
          }
  #pragma unroll
          for (int i = 0; i < TM; i++) {
            const int r = wm * WM + i * 32 + lr;
            const uint4 v = *reinterpret_cast<const uint4*>(qa + r * kRowBytes + Gm::swz(r, c) * 16);
            const v8i fa = v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
  #pragma unroll
            for (int jn = 0; jn < TN; jn++) {
              const int xa = (int)xa4[i][j / 2], xb = (int)xb4[jn][j / 2];
              if (j % 2 == 0)
                acc[i][jn] = kSwap ? __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                                         fb[jn], fa, acc[i][jn], 4, 4, 0, xb, 0, xa)
                                   : __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                                         fa, fb[jn], acc[i][jn], 4, 4, 0, xa, 0, xb);
              else
                acc[i][jn] = kSwap ? __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                                         fb[jn], fa, acc[i][jn], 4, 4, 2, xb, 2, xa)
                                   : __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                                         fa, fb[jn], acc[i][jn], 4, 4, 2, xa, 2, xb);
            }
          }
        }
      }
      __syncthreads();  // all waves are done with the ring before it is reused
    } else {
    Stage<BM, SK, NT> ra;
      Stage<BN, SK, NT> rb;
      load_stage<BM, SK, NT>(ra, p.A, p.SFA, amap, a_lim, K, 0, sc_aligned, tid);
      load_stage<BN, SK, NT>(rb, Wq, Ws, bmap, p.N, K, 0, sc_aligned, tid);
      store_stage<BM, SK, NT>(ra, smem, smem + kA + kB, tid);
      store_stage<BN, SK, NT>(rb, smem + kA, smem + kA + kB + BM * kRowScales, tid);
      __syncthreads();
  
      for (int s = 0; s < nst; s++) {
        const bool more = s + 1 < nst;
        if (more) {
          load_stage<BM, SK, NT>(ra, p.A, p.SFA, amap, a_lim, K, (s + 1) * SK, sc_aligned, tid);
          load_stage<BN, SK, NT>(rb, Wq, Ws, bmap, p.N, K, (s + 1) * SK, sc_aligned, tid);
        }
        const uint8_t* st = smem + (s & 1) * kStage;
        const uint8_t* qa = st;
        const uint8_t* qb = st + kA;
        const uint8_t* sa = st + kA + kB;
        const uint8_t* sb = sa + BM * kRowScales;
  #pragma unroll
        for (int j = 0; j < SK / 64; j++) {
          const int c = 2 * j + g;  // 16-byte chunk = K values 64j + 32g .. +32 of the stage
          v8i fb[TN];
          int xb[TN];
  #pragma unroll
          for (int i = 0; i < TN; i++) {
            const int r = wn * WN + i * 32 + lr;
            const uint4 v = *reinterpret_cast<const uint4*>(qb + r * kRowBytes + Gm::swz(r, c) * 16);
            fb[i] = v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
            xb[i] = sb[r * kRowScales + c];
          }
  #pragma unroll
          for (int i = 0; i < TM; i++) {
            const int r = wm * WM + i * 32 + lr;
            const uint4 v = *reinterpret_cast<const uint4*>(qa + r * kRowBytes + Gm::swz(r, c) * 16);
            const v8i fa = v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
            const int xa = sa[r * kRowScales + c];
  #pragma unroll
            for (int jn = 0; jn < TN; jn++)
              acc[i][jn] = kSwap ? __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[jn], fa, acc[i][jn], 4, 4, 0,
                                                                                   xb[jn], 0, xa)
                                 : __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa, fb[jn], acc[i][jn], 4, 4, 0,
                                                                                   xa, 0, xb[jn]);
          }
        }
        if (more) {
          uint8_t* nx = smem + ((s + 1) & 1) * kStage;
          store_stage<BM, SK, NT>(ra, nx, nx + kA + kB, tid);
          store_stage<BN, SK, NT>(rb, nx + kA, nx + kA + kB + BM * kRowScales, tid);
        }
        __syncthreads();
      }
  
    }

    // ---- epilogues.  A first: acc[i][jn][r] = tile row wm*WM + 32i + 8(r/4) +
    //      4g + r%4, tile column wn*WN + 32jn + lr.  B first: acc[i][jn][r] =
    //      tile row wm*WM + 32i + lr, tile column wn*WN + 32jn + 8(r/4) + 4g + r%4.
    if constexpr (kDMA && EPI != kEpiSilu) {
      // the tile goes through LDS (the ring is free after the K loop's last
      // barrier): each lane writes its 4-column runs, then each store writes
      // 16 contiguous bytes per lane, whole row segments of BN columns
      if constexpr (EPI == kEpiCombine) {
        if (tid < BM) row_f[tid] = rf;
      }
#pragma unroll
      for (int i = 0; i < TM; i++) {
        const int r = wm * WM + i * 32 + lr;
#pragma unroll
        for (int jn = 0; jn < TN; jn++)
#pragma unroll
          for (int q = 0; q < 4; q++) {
            const int c = wn * WN + jn * 32 + 8 * q + 4 * g;
            uint8_t* dst = smem + r * kOutPitch + c * kOutElem;
            if constexpr (EPI == kEpiCombine)
              *reinterpret_cast<float4*>(dst) =
                  make_float4(acc[i][jn][4 * q], acc[i][jn][4 * q + 1], acc[i][jn][4 * q + 2], acc[i][jn][4 * q + 3]);
            else
              *reinterpret_cast<uint2*>(dst) =
                  make_uint2(pack_bf16x2(alpha * acc[i][jn][4 * q], alpha * acc[i][jn][4 * q + 1]),
                             pack_bf16x2(alpha * acc[i][jn][4 * q + 2], alpha * acc[i][jn][4 * q + 3]));
          }
      }
      __syncthreads();
      constexpr int kChunksPerRow = BN * kOutElem / 16;
      for (int idx = tid; idx < BM * kChunksPerRow; idx += NT) {
        const int r = idx / kChunksPerRow, cb = (idx % kChunksPerRow) * 16;  // byte offset in the row
        const int n = tn * BN + cb / kOutElem;
        if (n >= p.N) continue;
        const uint4 v = *reinterpret_cast<const uint4*>(smem + r * kOutPitch + cb);
        if constexpr (EPI == kEpiCombine) {
          // y[f] = row, f = flat (token, slot) index of the row; the weighted
          // top-k sum is done afterwards in a fixed order (no atomics)
          const int f = row_f[r];
          if (f >= 0) *reinterpret_cast<uint4*>(p.y_f32 + (int64_t)f * p.N + n) = v;
        } else {
          const int m = m0 + r;
          if (m < nvalid_a) *reinterpret_cast<uint4*>(p.out + (int64_t)m * p.N + n) = v;
        }
      }
    } else if constexpr (EPI == kEpiStore) {
#pragma unroll
      for (int i = 0; i < TM; i++)
#pragma unroll
        for (int jn = 0; jn < TN; jn++) {
          const int n = tn * BN + wn * WN + jn * 32 + lr;
#pragma unroll
          for (int r = 0; r < 16; r++) {
            const int m = m0 + wm * WM + i * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
            if (m < nvalid_a && n < p.N)
              p.out[(int64_t)m * p.N + n] = (uint16_t)float_to_bf16_rne(alpha * acc[i][jn][r]);
          }
        }
    } else if constexpr (EPI == kEpiCombine) {
      // y[f] = row, f = flat (token, slot) index of the row; the weighted top-k
      // sum is done afterwards in a fixed order (deterministic, no atomics)
      if (tid < BM) row_f[tid] = rf;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < TM; i++) {
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const int m = m0 + wm * WM + i * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          if (m >= nvalid_a) continue;
          const int f = row_f[wm * WM + i * 32 + 8 * (r >> 2) + 4 * g + (r & 3)];
          float* dst = p.y_f32 + (int64_t)f * p.N;
#pragma unroll
          for (int jn = 0; jn < TN; jn++) {
            const int n = tn * BN + wn * WN + jn * 32 + lr;
            if (n < p.N) dst[n] = acc[i][jn][r];
          }
        }
      }
    } else {
      // SILU: gate tile 2jp and up tile 2jp+1 hold the same act columns, so a
      // lane has act values 8q + 4g + t (q, t < 4) of act block
      // b = tn*(BN/64) + wn*(TN/2) + jp of row m, and lane l ^ 32 the other 16.
      // act = bf16(silu(h_g) * h_u) from the bf16-rounded h (SiLU with the
      // hardware exp2 and reciprocal); the block's amax is shared between the
      // two lanes, E8M0 scale = smallest power of two >= amax / 6, E2M1 codes of
      // value / scale two at a time; each lane assembles 8 of the block's 16
      // code bytes with its partner's help and stores them.
      constexpr float kLog2e = 1.4426950408889634f;
      const int act_w = p.N / 2;
#pragma unroll
      for (int i = 0; i < TM; i++) {
        const int m = m0 + wm * WM + i * 32 + lr;
#pragma unroll
        for (int jp = 0; jp < TN / 2; jp++) {
          const int b = tn * (BN / 64) + wn * (TN / 2) + jp;  // act block index
          if (m >= nvalid_a || 32 * b >= act_w) continue;      // same for lanes l and l ^ 32
          float a[16];
          float amax = 0.0f;
#pragma unroll
          for (int r = 0; r < 16; r++) {
            const bf16x2 h = bf16x2{(__bf16)acc[i][2 * jp][r], (__bf16)acc[i][2 * jp + 1][r]};
            const float hg = (float)h.x, hu = (float)h.y;
            const float e = __builtin_amdgcn_exp2f(-hg * kLog2e);
            a[r] = (float)(__bf16)(hg * __builtin_amdgcn_rcpf(1.0f + e) * hu);
            amax = fmaxf(amax, fabsf(a[r]));
          }
          amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
          const uint32_t sc = e8m0_ceil(amax / 6.0f);
          // piece q: codes of columns 8q + 4g .. +3 (two bytes, first column in the low nibble)
          uint32_t piece[4];
#pragma unroll
          for (int q = 0; q < 4; q++) {
            uint32_t w2 = 0;
            w2 = e2m1x2_f32_pow2(w2, a[4 * q], a[4 * q + 1], sc, 0);
            w2 = e2m1x2_f32_pow2(w2, a[4 * q + 2], a[4 * q + 3], sc, 1);
            piece[q] = w2 & 0xFFFFu;
          }
          // block dword q = piece q of lane g = 0 | piece q of lane g = 1 << 16;
          // lane g = 0 writes dwords 0, 1 and lane g = 1 dwords 2, 3
          const uint32_t give = g == 0 ? (piece[2] | (piece[3] << 16)) : (piece[0] | (piece[1] << 16));
          const uint32_t got = (uint32_t)__shfl_xor((int)give, 32, 64);
          const uint2 out = g == 0 ? make_uint2(piece[0] | ((got & 0xFFFFu) << 16), piece[1] | (got & 0xFFFF0000u))
                                   : make_uint2((got & 0xFFFFu) | (piece[2] << 16), (got >> 16) | (piece[3] << 16));
          *reinterpret_cast<uint2*>(p.out_q + (int64_t)m * (act_w / 2) + b * 16 + 8 * g) = out;
          if (g == 0) p.out_sf[(int64_t)m * (act_w / 32) + b] = (uint8_t)sc;
        }
      }
    }
    __syncthreads();  // LDS is reused by the next work item
  }
}


// Loader waves of the DMA ring (BSFP4_MXFP4_LOADERS, measurement override):
// 0 = every wave issues its share.
int loaders() {
  const char* e = getenv("BSFP4_MXFP4_LOADERS");
  return e ? atoi(e) : 0;
}

// Ring form: 256-value stages in a 2-slot ring when K % 256 == 0 (whole
// 128-byte rows per DMA request; measured 92 -> 74 us on the 4096 x 4096 x 7168
// dense GEMM and 163 -> 145 / 130 -> 124 us on the MoE gate_up / down GEMMs
// against 128-value stages in 4 slots, while 3 slots of 256 values, which
// leave one workgroup per CU, measured slower), else 128-value stages in 4
// slots.  Measurement override BSFP4_MXFP4_RING = "128x4", "256x2" or "256x3".
int ring_form(int def) {
  const char* e = getenv("BSFP4_MXFP4_RING");
  if (!e) return def;
  if (!strcmp(e, "128x4")) return 0;
  if (!strcmp(e, "256x2")) return 1;
  if (!strcmp(e, "256x3")) return 2;
  return def;
}

template <int BM, int BN, int WGN, int EPI, int SK, int RING, int LOADERS>
hipError_t launch_ring(const Args& a, int64_t max_items, hipStream_t stream) {
  if constexpr (RING > 2 && ring_lds_bytes<BM, BN, SK, RING>() + 4096 > 160 * 1024) {
    // a deeper ring of this tile does not fit in LDS: two slots
    return launch_ring<BM, BN, WGN, EPI, SK, 2, LOADERS>(a, max_items, stream);
  } else {
    constexpr int NT = 128 * WGN;
    int64_t grid = (int64_t)device_cu_count() * wg_per_cu<BM, BN, SK, RING>();
    if (max_items < grid) grid = max_items < 1 ? 1 : max_items;
    if constexpr (chunked_scales<SK, RING>()) {
      if ((a.K / 32) % 16 == 0) {  // 16-byte-aligned scale rows: 16-byte lanes for the scale chunks
        mxfp4_grouped<BM, BN, WGN, SK, EPI, true, LOADERS, RING, true><<<(unsigned)grid, NT, 0, stream>>>(a);
        return hipGetLastError();
      }
    }
    mxfp4_grouped<BM, BN, WGN, SK, EPI, true, LOADERS, RING><<<(unsigned)grid, NT, 0, stream>>>(a);
    return hipGetLastError();
  }
}

template <int BM, int BN, int WGN, int SK, int EPI>
hipError_t launch(const Args& a, int64_t max_items, hipStream_t stream) {
  constexpr int NT = 128 * WGN;
  if (a.K % 128 == 0) {
    int form = ring_form(a.K % 256 == 0 ? 1 : 0);
    if (form != 0 && a.K % 256 != 0) form = 0;
    if (form == 1) return launch_ring<BM, BN, WGN, EPI, 256, 2, 0>(a, max_items, stream);
    if (form == 2) return launch_ring<BM, BN, WGN, EPI, 256, 3, 0>(a, max_items, stream);
    const int l = loaders();
    if (l == 2 && (BM + BN) / 64 % 2 == 0) return launch_ring<BM, BN, WGN, EPI, 128, 4, 2>(a, max_items, stream);
    if (l == 4 && NT / 64 > 4 && (BM + BN) / 64 % 4 == 0)
      return launch_ring<BM, BN, WGN, EPI, 128, 4, (NT / 64 > 4 ? 4 : 0)>(a, max_items, stream);
    return launch_ring<BM, BN, WGN, EPI, 128, 4, 0>(a, max_items, stream);
  }
  int64_t grid = (int64_t)device_cu_count() * wg_per_cu<BM, BN, SK, 2>();
  if (max_items < grid) grid = max_items < 1 ? 1 : max_items;
  mxfp4_grouped<BM, BN, WGN, SK, EPI, false, 0, 2><<<(unsigned)grid, NT, 0, stream>>>(a);
  return hipGetLastError();
}

// Waves per workgroup of the dense 256x256 kernel: 8 (2 x 4, two per SIMD) by
// default, BSFP4_MXFP4_WAVES=4 for 2 x 2.
int dense_waves() {
  const char* e = getenv("BSFP4_MXFP4_WAVES");
  return (e && e[0] == '4') ? 4 : 8;
}

}  // namespace

hipError_t launch_mxfp4_gemm(const uint8_t* A, const uint8_t* SFA, const uint8_t* B, const uint8_t* SFB,
                             const float* alpha, uint16_t* D, int64_t M, int64_t N, int64_t K,
                             hipStream_t stream) {
  if (M == 0) return hipSuccess;
  Args a{};
  a.A = A; a.SFA = SFA; a.rows = (int)M; a.a_rows = nullptr; a.a_nrows = (int)M;
  a.offsets = nullptr; a.E = 1;
  a.W = B; a.WSF = SFB; a.N = (int)N; a.K = (int)K; a.alpha = alpha; a.out = D;
  const int64_t items = ((M + 255) / 256) * ((N + 255) / 256);
  if (dense_waves() == 4) return launch<256, 256, 2, 128, kEpiStore>(a, items, stream);
  return launch<256, 256, 4, 128, kEpiStore>(a, items, stream);
}

hipError_t launch_mxfp4_grouped(const uint8_t* Aq, const uint8_t* Asf, const int32_t* a_rows, int64_t a_nrows,
                                const int32_t* offsets, int64_t E, int64_t rows, const uint8_t* W,
                                const uint8_t* Wsf, int64_t N, int64_t K, int epilogue, uint16_t* out,
                                uint8_t* out_q, uint8_t* out_sf, const int32_t* sorted_ids,
                                float* y_f32, hipStream_t stream) {
  Args a{};
  a.A = Aq; a.SFA = Asf; a.rows = (int)rows; a.a_rows = a_rows; a.a_nrows = (int)a_nrows;
  a.offsets = offsets; a.E = (int)E;
  a.W = W; a.WSF = Wsf; a.N = (int)N; a.K = (int)K; a.alpha = nullptr;
  a.out = out; a.out_q = out_q; a.out_sf = out_sf;
  a.sorted_ids = sorted_ids; a.y_f32 = y_f32;
  constexpr int BM = 128, BN = 128;
  const int64_t max_items = ((rows + BM - 1) / BM + E) * ((N + BN - 1) / BN);
  switch (epilogue) {
    case kEpiStore: return launch<BM, BN, 2, 128, kEpiStore>(a, max_items, stream);
    case kEpiSilu: return launch<BM, BN, 2, 128, kEpiSilu>(a, max_items, stream);
    default: return launch<BM, BN, 2, 128, kEpiCombine>(a, max_items, stream);
  }
}

}  // namespace bsfp4

// Host-side launchers of the gfx950 kernels (internal to libbsfp4).  Each
// assumes its arguments were validated by the C ABI layer and launches on
// the given stream; it returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bsfp4 {

// Compute units of the current device (cached on first use; 256 if the query fails).
int device_cu_count();

constexpr int64_t kQuantMaxGrid = 4096;
constexpr int64_t kAmaxMaxParts = 1024;

hipError_t launch_quantize(int fmt, const uint16_t* x, int64_t rows_in, int64_t K, const float* gs,
                           const int32_t* row_map, int64_t rows_out, uint8_t* q, uint8_t* sf,
                           hipStream_t stream);
// NVFP4 rows grouped by expert, row r of expert e quantised with gs[e].
hipError_t launch_nvfp4_experts_quant(const uint16_t* x, int64_t rows_in, int64_t K, const int32_t* row_map,
                                      const int32_t* offsets, int64_t E, const float* gs, int64_t rows_out,
                                      uint8_t* q, uint8_t* sf, hipStream_t stream);

// The library's static device scratch (scratch.hip): kScratchBytes per device,
// its address for the current device looked up once and cached.
constexpr size_t kScratchBytes = (size_t)32 << 20;
hipError_t scratch_device_ptr(void** out);

// Peak probes (probes.hip): MFMA loop per kind on probe_mfma_grid() workgroups
// of 256 threads, and a 128-bit streaming read of `bytes` (bytes % 16 == 0).
int64_t probe_mfma_grid();
hipError_t launch_probe_mfma(int kind, int iters, hipStream_t stream);
hipError_t launch_probe_read(const void* buf, int64_t bytes, hipStream_t stream);

// E2M1 codes of caller-given value pairs (see bsfp4_e2m1_convert); pairs % 4 == 0.
hipError_t launch_e2m1_convert(int mode, const void* in, const uint8_t* scale_codes, int64_t pairs,
                               uint8_t* codes, hipStream_t stream);

int global_scale_parts(int64_t numel);
hipError_t launch_global_scale(const uint16_t* x, int64_t numel, float* gs, float* partial,
                               hipStream_t stream);

hipError_t launch_nvfp4_gemm(const uint8_t* A, const uint8_t* SFA, const uint8_t* B, const uint8_t* SFB,
                             const float* alpha, uint16_t* D, int64_t M, int64_t N, int64_t K,
                             void* ws, size_t ws_bytes, hipStream_t stream);
size_t nvfp4_gemm_workspace(int64_t M, int64_t N, int64_t K);

// Small-M (M <= 64) kernels with NVFP4 weights.  Some forms split K over work
// items and need `part` = skinny_workspace(M, N, K, activations are NVFP4)
// bytes of FP32 partials (nullptr when that is 0).
constexpr int64_t kSkinnyMaxM = 64;
hipError_t launch_skinny_nvfp4(const uint8_t* A, const uint8_t* SFA, const uint8_t* B, const uint8_t* SFB,
                               const float* alpha, uint16_t* D, int64_t M, int64_t N, int64_t K, float* part,
                               hipStream_t stream);
hipError_t launch_skinny_w4a16(const uint16_t* A, const uint8_t* B, const uint8_t* SFB, const float* alpha,
                               uint16_t* D, int64_t M, int64_t N, int64_t K, float* part, hipStream_t stream);
size_t skinny_workspace(int64_t M, int64_t N, int64_t K, bool fp4_activations);

// Tiled W4A16 for M > kSkinnyMaxM (K % 64 == 0, operands below 2^31 bytes).
bool w4a16_tiled_ok(int64_t M, int64_t N, int64_t K);
size_t w4a16_tiled_workspace(int64_t M, int64_t N, int64_t K);
hipError_t launch_w4a16_tiled(const uint16_t* A, const uint8_t* B, const uint8_t* SFB, const float* alpha,
                              uint16_t* D, int64_t M, int64_t N, int64_t K, float* part, size_t part_bytes,
                              hipStream_t stream);
// W4A16 for 33..64 rows (K % 128 == 0): 64 x 128 tiles over K ranges.
bool w4a16_rows64_ok(int64_t M, int64_t N, int64_t K);
size_t w4a16_rows64_workspace(int64_t M, int64_t N, int64_t K);
hipError_t launch_w4a16_rows64(const uint16_t* A, const uint8_t* B, const uint8_t* SFB, const float* alpha,
                               uint16_t* D, int64_t M, int64_t N, int64_t K, float* part, size_t part_bytes,
                               hipStream_t stream);
// The same 64-row kernel with NVFP4 activations (fp16 MFMA); its K split and
// workspace are those of the W4A16 form (w4a16_rows64_workspace).
bool nvfp4_rows64_ok(int64_t M, int64_t N, int64_t K);
hipError_t launch_nvfp4_rows64(const uint8_t* A, const uint8_t* SFA, const uint8_t* B, const uint8_t* SFB,
                               const float* alpha, uint16_t* D, int64_t M, int64_t N, int64_t K, float* part,
                               size_t part_bytes, hipStream_t stream);
// D = bf16(alpha * sum_s part[s]) over `splits` FP32 partials of MN elements
// (MN % 4 == 0), summed in split order.
hipError_t launch_splitk_reduce(const float* part, int splits, const float* alpha, uint16_t* D, int64_t MN,
                                hipStream_t stream);

// Row-major [rows, kblocks] scales <-> padded 128x4 swizzled layout (0: SM100
// form, 1: SM103 form); to_swizzled chooses the direction.
hipError_t launch_scale_layout(int layout, bool to_swizzled, const uint8_t* src, uint8_t* dst, int64_t rows,
                               int64_t kblocks, hipStream_t stream);

// MXFP4 scaled-MFMA GEMMs (dense and grouped by expert).
constexpr int kEpiStore = 0;    // bf16 rows
constexpr int kEpiSilu = 1;     // SiLU(gate) * up, re-quantised to MXFP4
constexpr int kEpiCombine = 2;  // top-k weighted FP32 accumulation into token rows
constexpr int64_t kMaxExperts = 1024;
hipError_t launch_mxfp4_gemm(const uint8_t* A, const uint8_t* SFA, const uint8_t* B, const uint8_t* SFB,
                             const float* alpha, uint16_t* D, int64_t M, int64_t N, int64_t K,
                             hipStream_t stream);
hipError_t launch_mxfp4_grouped(const uint8_t* Aq, const uint8_t* Asf, const int32_t* a_rows, int64_t a_nrows,
                                const int32_t* offsets, int64_t E, int64_t rows, const uint8_t* W,
                                const uint8_t* Wsf, int64_t N, int64_t K, int epilogue, uint16_t* out,
                                uint8_t* out_q, uint8_t* out_sf, const int32_t* sorted_ids,
                                float* y_f32, hipStream_t stream);

// Fused NVFP4 quantise + GEMM for at most four rows (the bf16 rows quantised
// with gs inside every workgroup; the same D as fp4_quantize then the GEMM).
bool nvfp4_fused_quant_gemm_ok(int64_t M, int64_t N, int64_t K);
hipError_t launch_nvfp4_fused_quant_gemm(const uint16_t* x, const float* gs, const uint8_t* B, const uint8_t* SFB,
                                         const float* alpha, uint16_t* D, int64_t M, int64_t N, int64_t K,
                                         hipStream_t stream);

// NVFP4 grouped GEMM over per-expert weights, fp16-dequant core (epilogues as
// above; SILU re-quantises to NVFP4 with the per-expert global scale out_gs).
hipError_t launch_nvfp4_grouped(const uint8_t* Aq, const uint8_t* Asf, const int32_t* offsets, int64_t E,
                                int64_t rows, const uint8_t* W, const uint8_t* Wsf, const float* alpha,
                                int64_t N, int64_t K, int epilogue, uint16_t* out, uint8_t* out_q, uint8_t* out_sf,
                                const float* out_gs, const int32_t* sorted_ids, float* y, hipStream_t stream);

// MoE routing prep and the combine's helpers.
hipError_t launch_moe_prep(const int32_t* topk_ids, int64_t T, int64_t topk, int64_t E, int32_t* offsets,
                           int32_t* sorted_ids, int32_t* sorted_tokens, hipStream_t stream);
hipError_t launch_topk_sum(const float* y, const float* w, uint16_t* out, int64_t T, int64_t topk, int64_t N,
                           hipStream_t stream);

}  // namespace bsfp4

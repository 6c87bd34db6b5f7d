/*
 * bsfp4.h -- block-scaled FP4 (E2M1) kernels for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libbsfp4.so.  Every entry point takes plain device pointers,
 * element counts and a HIP stream passed as `void*` (a hipStream_t; NULL
 * means the null stream).  No entry point allocates, frees or synchronises:
 * the caller owns every buffer (inputs, outputs and workspace) and every
 * call is asynchronous on the given stream.  Device-side faults surface at
 * the caller's next synchronisation, as with any HIP call.
 *
 * Data formats (as named on the pages this library implements):
 *   E2M1   4-bit float, values {0, 0.5, 1, 1.5, 2, 3, 4, 6} and negatives.
 *          Packed two per byte along K; element 2j sits in the low nibble of
 *          byte j (vLLM `sm103` branch comparison page,
 *          `nvfp4_quant_kernels.cu`, `cvt_fp16_to_fp4_sm103`: the first
 *          elements of a thread land in the low bits of the packed word).
 *   E4M3   8-bit scale (OCP "fn": bias 7, max 448, NaN at 0x7F/0xFF); one
 *          per 16 K-elements in the NVFP4 form (`float_ue4m3_t` block scales
 *          of `Fp4GemmSm103`, same page, `nvfp4_scaled_mm_kernels.cu`).
 *   E8M0   8-bit power-of-two scale 2^(c-127); one per 32 K-elements in the
 *          MXFP4 form ("[Kernel] Enable CUTLASS MXFP4 W4A4 MoE on SM12x").
 *   bf16   activations and outputs, passed as 16-bit patterns.
 * Scale tensors are row-major [rows, K/16] (NVFP4) or [rows, K/32] (MXFP4),
 * one byte per block, unpadded and unswizzled.  Codes are row-major
 * [rows, K/2].  Every matrix is contiguous.
 *
 * Errors: each call validates its arguments before any launch and returns a
 * status; on error nothing is launched and bsfp4_last_error() returns a
 * message for the calling thread.  Pointers must be 16-byte aligned
 * (128-bit vector loads and stores), except the scalar `gs`/`alpha`
 * pointers (4-byte aligned).  The extent of a buffer cannot be checked
 * through a pointer: the caller must pass buffers of exactly the documented
 * sizes (the Python binding checks them).
 *
 * State and thread safety: all entry points are thread-safe.  Besides the
 * per-thread error message, the library caches two fixed properties per
 * device id (whether it is a gfx950, and its compute-unit count), each filled
 * on first use without a data race.  The kernel planners also read BSFP4_*
 * environment variables on every call; these are measurement and test
 * overrides that force a particular kernel, tile or K split (results stay
 * within the documented tolerance whichever is chosen) and are unset in
 * normal use.
 */
#ifndef BSFP4_H_
#define BSFP4_H_

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define BSFP4_API __attribute__((visibility("default")))
#else
#define BSFP4_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum bsfp4_status {
  BSFP4_OK = 0,
  BSFP4_ERR_INVALID_ARG = 1, /* null pointer, unknown enum, negative size */
  BSFP4_ERR_SHAPE = 2,       /* a size violates a divisibility or range rule */
  BSFP4_ERR_ALIGNMENT = 3,   /* a pointer is not 16-byte (scalars: 4-byte) aligned */
  BSFP4_ERR_WORKSPACE = 4,   /* workspace missing or smaller than required */
  BSFP4_ERR_DEVICE = 5,      /* the current device is not a gfx950 GPU */
  BSFP4_ERR_HIP = 6          /* a HIP launch or runtime call failed */
} bsfp4_status;

typedef enum bsfp4_format {
  BSFP4_NVFP4 = 0, /* E2M1 values, E4M3 scale per 16 elements, FP32 global scale */
  BSFP4_MXFP4 = 1  /* E2M1 values, E8M0 scale per 32 elements */
} bsfp4_format;

/* Library version (major*10000 + minor*100 + patch). */
BSFP4_API int bsfp4_version(void);
/* Static description of a status code. */
BSFP4_API const char* bsfp4_status_string(int status);
/* Message of the last failed call on the calling thread ("" if none). */
BSFP4_API const char* bsfp4_last_error(void);

/* ----------------------------------------------------------------------------
 * fp4_global_scale: gs = 2688 / max|x| over a bf16 tensor (448 * 6 =
 * FLOAT8_E4M3_MAX * FLOAT4_E2M1_MAX; vLLM `sm103` branch comparison page,
 * `test_nvfp4_quant.py`, `test_scaled_fp4_quant_sm103_matches_sm100`).
 *   x        device, numel bf16 values (16-byte aligned)
 *   gs_out   device, one float written with fl32(2688 / amax); amax == 0
 *            gives +inf (the caller must not quantise an all-zero tensor
 *            with it)
 *   ws       device workspace of fp4_global_scale_workspace_size(numel) bytes
 * ------------------------------------------------------------------------- */
BSFP4_API size_t fp4_global_scale_workspace_size(int64_t numel);
BSFP4_API bsfp4_status fp4_global_scale(const uint16_t* x, int64_t numel, float* gs_out, void* ws,
                              size_t ws_bytes, void* stream);

/* ----------------------------------------------------------------------------
 * fp4_quantize: bf16 rows -> packed E2M1 codes + block scales.
 * Defines the activation quantiser `cvt_fp16_to_fp4_sm103` (vLLM `sm103`
 * branch comparison page, `nvfp4_quant_kernels.cu`) and the per-expert
 * MXFP4 activation quant (`mxfp4_experts_quant`, "[Kernel] Enable CUTLASS
 * MXFP4 W4A4 MoE on SM12x").  Per block of 16 (NVFP4) or 32 (MXFP4)
 * elements v along a row:
 *   NVFP4: s = fl32(fl32(amax/6) * gs); sf = E4M3 round-to-nearest-even of
 *          s, saturating at 448; inv = fl32(gs / dec(sf)) (0 if dec(sf)==0)
 *   MXFP4: sf = E8M0 of the smallest power of two >= fl32(amax/6);
 *          inv = 2^(127-sf)
 *   code  = E2M1 round-to-nearest-even of fl32(v * inv), saturating at 6,
 *           sign bit kept (negative values that round to 0 give code 8).
 *   fmt       BSFP4_NVFP4 or BSFP4_MXFP4
 *   x         device bf16 [rows_in, K]
 *   K         row length; K % 16 == 0 (NVFP4) or K % 32 == 0 (MXFP4), K > 0
 *   gs        device float[1]; required for NVFP4, must be NULL for MXFP4
 *   row_map   device int32[rows_out] or NULL.  If given, output row r
 *             quantises input row row_map[r] (0 <= row_map[r] < rows_in;
 *             out-of-range entries produce all-zero rows).  NULL means
 *             rows_out == rows_in and row r -> row r.
 *   q         device uint8 [rows_out, K/2]
 *   sf        device uint8 [rows_out, K/16] or [rows_out, K/32]
 * rows_out == 0 is a valid no-op.
 * ------------------------------------------------------------------------- */
BSFP4_API bsfp4_status fp4_quantize(int fmt, const uint16_t* x, int64_t rows_in, int64_t K,
                          const float* gs, const int32_t* row_map, int64_t rows_out,
                          uint8_t* q, uint8_t* sf, void* stream);

/* ----------------------------------------------------------------------------
 * fp4_gemm: D[M,N] = bf16_rne(alpha * sum_k dec(A)[m,k] * dec(B)[n,k]).
 * The W4A4 block-scaled GEMM of `Fp4GemmSm103` / `cutlass_scaled_fp4_mm`
 * (vLLM `sm103` branch comparison page, `nvfp4_scaled_mm_kernels.cu` and
 * `nvfp4_scaled_mm_entry.cu`) and CuTe-DSL `mm_fp4` ("perf(gemm): optimize
 * SM103 CuTe DSL mm_fp4 kernel"); alpha multiplies the FP32 accumulator and
 * the result is converted to bf16 once (that page, "Alpha epilogue bug").
 *   fmt       BSFP4_NVFP4 (E4M3 scales per 16) or BSFP4_MXFP4 (E8M0 per 32)
 *   A, SFA    device [M, K/2] codes, [M, K/16 or K/32] scales
 *   B, SFB    device [N, K/2] codes, [N, K/16 or K/32] scales (row n holds
 *             output column n's weights, contiguous along K)
 *   alpha     device float[1]; NULL means 1.0
 *   D         device bf16 [M, N]
 *   sizes     M >= 0, N % 32 == 0, K % 32 == 0, N > 0, K > 0 (the pages'
 *             `cutlass_scaled_fp4_mm_sm103a_impl` checks); for MXFP4 also
 *             M*K/2 < 2^31 and N*K/2 < 2^31 (32-bit buffer offsets),
 *             otherwise BSFP4_ERR_SHAPE
 *   ws        device workspace of fp4_gemm_workspace_size(...) bytes (may be
 *             NULL when that size is 0); its contents need no initialisation
 * NVFP4 block scales are non-negative, as fp4_quantize writes them: the
 * kernels read an E4M3 scale's 7 magnitude bits only, and the NaN codes
 * (0x7F, 0xFF) are outside the contract.
 * Results equal the float64 definition up to FP32 summation order.
 * ------------------------------------------------------------------------- */
BSFP4_API size_t fp4_gemm_workspace_size(int fmt, int64_t M, int64_t N, int64_t K);
BSFP4_API bsfp4_status fp4_gemm(int fmt, const uint8_t* A, const uint8_t* SFA, const uint8_t* B,
                      const uint8_t* SFB, const float* alpha, uint16_t* D, int64_t M, int64_t N,
                      int64_t K, void* ws, size_t ws_bytes, void* stream);

/* ----------------------------------------------------------------------------
 * fp4_gemm_noalloc: fp4_gemm without a workspace argument, for callers that
 * cannot allocate device memory at all (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).  The split-K partials
 * that fp4_gemm keeps in the caller's workspace go to a static device array
 * of the library instead, fp4_gemm_noalloc_max_workspace() bytes (32 MiB) on
 * every GPU the library runs on, held until the process ends; the call
 * itself allocates and frees nothing and issues no memset.
 *   arguments, layouts and results as for fp4_gemm (the same kernels, tile
 *   plan and K split, so the output equals fp4_gemm's bit for bit)
 *   returns BSFP4_ERR_WORKSPACE, before any launch, when the shape needs
 *   more than fp4_gemm_noalloc_max_workspace() bytes of partials, i.e. when
 *   fp4_gemm_workspace_size(fmt, M, N, K) exceeds it (NVFP4 with M = 1024 at
 *   N = 4096, K = 7168, for example; MXFP4 never needs any)
 * Every call on one GPU shares that GPU's array, and the partials of a call
 * are written in full before they are read, so nothing needs clearing; calls
 * that overlap in time on one GPU (different streams, or threads) race on
 * the array and must be serialised by the caller.
 * ------------------------------------------------------------------------- */
BSFP4_API size_t fp4_gemm_noalloc_max_workspace(void);
BSFP4_API bsfp4_status fp4_gemm_noalloc(int fmt, const uint8_t* A, const uint8_t* SFA, const uint8_t* B,
                                        const uint8_t* SFB, const float* alpha, uint16_t* D, int64_t M,
                                        int64_t N, int64_t K, void* stream);

/* ----------------------------------------------------------------------------
 * w4a16_gemm: D[M,N] = bf16_rne(alpha * sum_k A[m,k] * dec(B)[n,k]) with bf16
 * activations and NVFP4 weights ("feat: sm100 cute_dsl w4a16 gemm": bf16
 * activations x native NVFP4 weights; the tensor-wide FP32 weight scale
 * multiplies the FP32 accumulator in the epilogue).
 *   A         device bf16 [M, K]
 *   B, SFB    device [N, K/2] E2M1 codes, [N, K/16] E4M3 scales
 *   alpha     device float[1]; NULL means 1.0
 *   D         device bf16 [M, N]
 *   sizes     M >= 0, N % 32 == 0, K % 32 == 0
 *   ws        device workspace of w4a16_gemm_workspace_size(...) bytes (may
 *             be NULL when that size is 0); its contents need no
 *             initialisation
 * Block scales follow fp4_gemm's rule (non-negative, no NaN codes).  Results
 * equal the float64 definition up to FP32 summation order.
 * ------------------------------------------------------------------------- */
BSFP4_API size_t w4a16_gemm_workspace_size(int64_t M, int64_t N, int64_t K);
BSFP4_API bsfp4_status w4a16_gemm(const uint16_t* A, const uint8_t* B, const uint8_t* SFB,
                        const float* alpha, uint16_t* D, int64_t M, int64_t N, int64_t K,
                        void* ws, size_t ws_bytes, void* stream);

/* ----------------------------------------------------------------------------
 * Block-scale layout interchange.  This library keeps block scales row-major,
 * one byte per block ([rows, K/16] E4M3 or [rows, K/32] E8M0); the pages'
 * block-scaled GEMMs take them padded to [round_up(rows, 128),
 * round_up(kblocks, 4)] and swizzled in 512-byte tiles of 128 rows x 4
 * columns, tile (row tile, column tile) at (row_tile * column_tiles +
 * column_tile) * 512, the 4 columns of a tile's local row r consecutive at
 *   BSFP4_SF_128X4     (the SM100 form, also read as the 6-D view
 *                      (32, 4, rows/128, 4, kblocks/4, 1) of the W4A16 pages):
 *                      (r % 32) * 16 + (r / 32) * 4
 *   BSFP4_SF_128X4_M8  (the SM103 form): (r / 16) * 16 + ((r / 4) % 4) * 128
 *                      + (r % 4) * 4
 * (vLLM `sm103` branch comparison page, `nvfp4_quant_kernels.cu`: the SM103
 * scale-offset helper and the SM100 <-> SM103 conversion kernel;
 * `nvfp4_scaled_mm_entry.cu`: the padded shape checks).  Padding bytes are
 * written as zeros.  These calls import and export that layout so that scales
 * prepared for the pages' kernels can be used here and vice versa.
 *   rows, kblocks  rows >= 0, kblocks > 0, padded size below 2^31 bytes
 *   sf             device row-major [rows, kblocks] bytes (any alignment)
 *   swz            device [round_up(rows,128), round_up(kblocks,4)] bytes,
 *                  4-byte aligned; fp4_scales_swizzled_size() bytes
 * Byte-exact permutations; nothing is allocated.
 * ------------------------------------------------------------------------- */
typedef enum bsfp4_sf_layout {
  BSFP4_SF_128X4 = 0,
  BSFP4_SF_128X4_M8 = 1
} bsfp4_sf_layout;

BSFP4_API size_t fp4_scales_swizzled_size(int64_t rows, int64_t kblocks);
BSFP4_API bsfp4_status fp4_scales_swizzle(int layout, const uint8_t* sf, int64_t rows, int64_t kblocks,
                                          uint8_t* swz, void* stream);
BSFP4_API bsfp4_status fp4_scales_unswizzle(int layout, const uint8_t* swz, int64_t rows, int64_t kblocks,
                                            uint8_t* sf, void* stream);

/* ----------------------------------------------------------------------------
 * fp4_moe_prep: group routed (token, slot) pairs by expert.  Produces the
 * per-expert row offsets that the pages' experts ops take
 * (`input_offset_by_experts`, vLLM `sm103` branch comparison page,
 * `csrc/ops.h`).
 *   topk_ids        device int32 [T, topk], each in [0, E)
 *   expert_offsets  device int32 [E+1]: rows of expert e are
 *                   [offsets[e], offsets[e+1]); offsets[E] == T*topk
 *   sorted_ids      device int32 [T*topk]: flat index t*topk+j of each row,
 *                   stable within an expert (increasing flat index)
 *   sorted_tokens   device int32 [T*topk] or NULL: token t = sorted_ids/topk
 *                   of each row (the row_map of the experts quantiser)
 *   ws              device workspace of fp4_moe_prep_workspace_size bytes
 * Ids outside [0, E) are not checked on the device and give undefined
 * groupings (never out-of-bounds writes: they are dropped).
 * ------------------------------------------------------------------------- */
BSFP4_API size_t fp4_moe_prep_workspace_size(int64_t T, int64_t topk, int64_t E);
BSFP4_API bsfp4_status fp4_moe_prep(const int32_t* topk_ids, int64_t T, int64_t topk, int64_t E,
                          int32_t* expert_offsets, int32_t* sorted_ids,
                          int32_t* sorted_tokens, void* ws, size_t ws_bytes, void* stream);

/* ----------------------------------------------------------------------------
 * mxfp4_moe_grouped_gemm: for every expert e, problem rows [off[e], off[e+1])
 * times expert e's MXFP4 weights ("[Kernel] Enable CUTLASS MXFP4 W4A4 MoE on
 * SM12x": MXFP4 x MXFP4 grouped GEMM over per-expert weights).  alpha is 1.
 * A persistent grid walks the list of (expert, column tile, row tile) items.
 *   Aq, Asf          device [a_rows_total, K/2] codes, [a_rows_total, K/32]
 *                    E8M0 scales
 *   a_row_index      device int32 [rows] or NULL: problem row m reads row
 *                    a_row_index[m] of Aq (e.g. the token of a sorted row, so
 *                    activations are quantised once per token); entries outside
 *                    [0, a_rows_total) read as zero.  NULL: row m reads row m
 *                    and a_rows_total must equal rows.
 *   expert_offsets   device int32 [E+1] (from fp4_moe_prep), 1 <= E <= 1024
 *   rows             problem rows (T*topk for a routed layer)
 *   W, Wsf           device [E, N, K/2], [E, N, K/32]
 *   N % 32 == 0 (N % 64 == 0 for SILU_MUL_QUANT), K % 32 == 0;
 *   a_rows_total*K/2 < 2^31 and N*K/2 < 2^31 (32-bit buffer offsets),
 *   otherwise BSFP4_ERR_SHAPE
 *   epilogue         one of bsfp4_moe_epilogue; its fields in `ep`:
 *     BSFP4_MOE_STORE_BF16:  ep.out = bf16 [rows, N]
 *     BSFP4_MOE_SILU_MUL_QUANT: act = bf16(silu(h[:, :N/2]) * h[:, N/2:])
 *         with h the bf16-rounded GEMM row, MXFP4-quantised into
 *         ep.out_q [rows, N/4] and ep.out_sf [rows, N/64] (the fused
 *         `silu_and_mul_scaled_fp4_experts_quant` pattern of the vLLM `sm103`
 *         branch comparison page, `csrc/ops.h`, in its MXFP4 form)
 *     BSFP4_MOE_WEIGHTED_COMBINE: ep.out = bf16 [T, N] with
 *         out[t] = bf16(sum_j w[t,j] * Y[row(t,j)]): each GEMM row is kept in
 *         FP32 (workspace, rows*N*4 bytes), then a token's top-k rows, each
 *         times its routing weight (FP32 product), are summed in slot order
 *         (deterministic); uses ep.sorted_ids, ep.topk_weights [T*topk],
 *         ep.num_tokens, ep.topk
 *   ws               device workspace of
 *                    mxfp4_moe_grouped_gemm_workspace_size(...) bytes
 * ------------------------------------------------------------------------- */
typedef enum bsfp4_moe_epilogue {
  BSFP4_MOE_STORE_BF16 = 0,
  BSFP4_MOE_SILU_MUL_QUANT = 1,
  BSFP4_MOE_WEIGHTED_COMBINE = 2
} bsfp4_moe_epilogue;

typedef struct bsfp4_moe_epilogue_args {
  void* out;                   /* bf16 output (STORE_BF16, WEIGHTED_COMBINE) */
  uint8_t* out_q;              /* MXFP4 codes of act (SILU_MUL_QUANT) */
  uint8_t* out_sf;             /* E8M0 scales of act (SILU_MUL_QUANT) */
  const int32_t* sorted_ids;   /* WEIGHTED_COMBINE */
  const float* topk_weights;   /* WEIGHTED_COMBINE, [num_tokens * topk] */
  int64_t num_tokens;          /* WEIGHTED_COMBINE */
  int64_t topk;                /* WEIGHTED_COMBINE */
  const float* out_gs;         /* nvfp4_moe_grouped_gemm SILU_MUL_QUANT: device
                                  float[E], global scale of act per expert;
                                  unused by mxfp4_moe_grouped_gemm */
} bsfp4_moe_epilogue_args;

BSFP4_API size_t mxfp4_moe_grouped_gemm_workspace_size(int64_t rows, int64_t E, int64_t N, int64_t K,
                                             int epilogue, int64_t num_tokens);
BSFP4_API bsfp4_status mxfp4_moe_grouped_gemm(const uint8_t* Aq, const uint8_t* Asf,
                                              int64_t a_rows_total, const int32_t* a_row_index,
                                              const int32_t* expert_offsets, int64_t E, int64_t rows,
                                              const uint8_t* W, const uint8_t* Wsf, int64_t N, int64_t K,
                                              int epilogue, const bsfp4_moe_epilogue_args* ep, void* ws,
                                              size_t ws_bytes, void* stream);

/* ----------------------------------------------------------------------------
 * nvfp4_quantize_gemm: the producer and consumer of a layer in one call,
 * D = fp4_gemm(NVFP4, fp4_quantize(NVFP4, x, gs), B, SFB, alpha), bit for bit
 * the output of the two-call sequence.  The HIP counterpart of the pages'
 * programmatic-dependent-launch overlap of `scaled_fp4_quant_sm103_pdl` and
 * `cutlass_scaled_fp4_mm_sm103a_pdl` (vLLM `sm103` branch comparison page,
 * "PDL" benchmarks of the quant + GEMM pair and the 4-layer pipeline): for up
 * to four rows (decode shapes, K <= 8192) every workgroup quantises the bf16
 * rows itself while its weight stream is in flight, so there is one kernel
 * and no intermediate buffer; otherwise the quantiser writes the codes and
 * scales into the workspace and the GEMM reads them.
 *   x       device bf16 [M, K]
 *   gs      device float[1], the activation global scale (e.g. from
 *           fp4_global_scale)
 *   B, SFB, alpha, D, M, N, K as for fp4_gemm with BSFP4_NVFP4
 *   ws      device workspace of nvfp4_quantize_gemm_workspace_size(M, N, K)
 *           bytes, 16-byte aligned (0 bytes on the fused path)
 * ------------------------------------------------------------------------- */
BSFP4_API size_t nvfp4_quantize_gemm_workspace_size(int64_t M, int64_t N, int64_t K);
BSFP4_API bsfp4_status nvfp4_quantize_gemm(const uint16_t* x, const float* gs, const uint8_t* B,
                                           const uint8_t* SFB, const float* alpha, uint16_t* D, int64_t M,
                                           int64_t N, int64_t K, void* ws, size_t ws_bytes, void* stream);

/* ----------------------------------------------------------------------------
 * NVFP4 mixture-of-experts layer: the per-expert NVFP4 ops the vLLM `sm103`
 * branch comparison page declares (`csrc/ops.h`, `torch_bindings.cpp`:
 * `scaled_fp4_experts_quant` and `silu_and_mul_scaled_fp4_experts_quant`,
 * both addressed through per-expert row offsets).  Every expert e carries its
 * own activation global scale and GEMM alpha (the dense NVFP4 conventions
 * applied per expert; the op bodies are not printed).
 *
 * nvfp4_experts_quantize: output row r (rows grouped by expert, as from
 * fp4_moe_prep) quantises input row row_map[r] (row r if row_map is NULL)
 * with the NVFP4 recipe of fp4_quantize, using gs_experts[e] for the expert e
 * with expert_offsets[e] <= r < expert_offsets[e+1].
 *   x            device bf16 [rows_in, K], K % 16 == 0
 *   row_map      device int32 [rows_out] or NULL (then rows_out == rows_in);
 *                entries outside [0, rows_in) give all-zero rows
 *   expert_offsets device int32 [E+1], 1 <= E <= 1024, non-decreasing; rows
 *                outside [offsets[0], offsets[E]) are written as zeros
 *   gs_experts   device float [E]
 *   q, sf        device uint8 [rows_out, K/2], [rows_out, K/16]
 * ------------------------------------------------------------------------- */
BSFP4_API bsfp4_status nvfp4_experts_quantize(const uint16_t* x, int64_t rows_in, int64_t K,
                                              const int32_t* row_map, const int32_t* expert_offsets,
                                              int64_t E, const float* gs_experts, int64_t rows_out,
                                              uint8_t* q, uint8_t* sf, void* stream);

/* ----------------------------------------------------------------------------
 * nvfp4_moe_grouped_gemm: for every expert e, rows [off[e], off[e+1]) of the
 * NVFP4 activations times expert e's NVFP4 weights, alpha_experts[e] applied
 * to the FP32 accumulator (`cutlass_fp4_group_mm` in the page's op list).
 * The products are exact (fp16 MFMA on the dequantised values) and accumulate
 * in FP32, as in fp4_gemm.
 *   Aq, Asf        device [rows, K/2] codes, [rows, K/16] E4M3 scales,
 *                  expert-sorted (e.g. from nvfp4_experts_quantize)
 *   expert_offsets device int32 [E+1], 1 <= E <= 1024
 *   W, Wsf         device [E, N, K/2], [E, N, K/16]; N*K/2 < 2^31
 *   alpha_experts  device float [E] or NULL (all 1.0)
 *   N % 32 == 0 (N % 64 == 0 for SILU_MUL_QUANT), K % 32 == 0
 *   epilogue       as for mxfp4_moe_grouped_gemm, except that
 *                  SILU_MUL_QUANT writes NVFP4: ep.out_q [rows, N/4] codes,
 *                  ep.out_sf [rows, N/32] E4M3 scales, act row of expert e
 *                  quantised with ep.out_gs[e] (the fused
 *                  `silu_and_mul_scaled_fp4_experts_quant`, NVFP4 form)
 *   ws             device workspace of
 *                  nvfp4_moe_grouped_gemm_workspace_size(...) bytes
 * Scales as for fp4_gemm: non-negative E4M3 codes.
 * ------------------------------------------------------------------------- */
BSFP4_API size_t nvfp4_moe_grouped_gemm_workspace_size(int64_t rows, int64_t E, int64_t N, int64_t K,
                                                       int epilogue, int64_t num_tokens);
BSFP4_API bsfp4_status nvfp4_moe_grouped_gemm(const uint8_t* Aq, const uint8_t* Asf,
                                              const int32_t* expert_offsets, int64_t E, int64_t rows,
                                              const uint8_t* W, const uint8_t* Wsf,
                                              const float* alpha_experts, int64_t N, int64_t K,
                                              int epilogue, const bsfp4_moe_epilogue_args* ep, void* ws,
                                              size_t ws_bytes, void* stream);

/* ----------------------------------------------------------------------------
 * Diagnostics.
 *
 * bsfp4_e2m1_convert: E2M1 codes of caller-given value pairs, computed by the
 * very device routines the quantiser kernels and the fused SiLU-mul + MXFP4
 * epilogue use (gfx950's v_cvt_scalef32_pk_fp4_* instructions), so that the
 * hardware rounding can be held to a reference encoder.  The pages name the
 * per-block routine (`cvt_warp_fp16_to_fp4`, `cvt_fp16_to_fp4_sm103`, vLLM
 * `sm103` branch comparison page, `nvfp4_quant_kernels.cu`) without printing
 * it; the rule implemented is nearest E2M1 value, ties to the even code,
 * saturation at 6, sign bit kept.
 *   mode         BSFP4_CVT_F32: `in` holds 2*pairs binary32 values (the
 *                NVFP4 quantiser's fl32(v * inv)), scale 1;
 *                BSFP4_CVT_BF16_E8M0: `in` holds 2*pairs bf16 values, pair i
 *                divided by 2^(scale_codes[i] - 127) (the MXFP4 quantiser);
 *                BSFP4_CVT_F32_E8M0: 2*pairs binary32 values, pair i divided
 *                by 2^(scale_codes[i] - 127) (the fused SiLU-mul epilogue)
 *   in           device, 16-byte aligned
 *   scale_codes  device uint8 [pairs] E8M0 codes 0..254 (NULL for
 *                BSFP4_CVT_F32), 16-byte aligned
 *   pairs        >= 0, a multiple of 4
 *   codes        device uint8 [pairs]: byte i = code of value 2i (low nibble)
 *                | code of value 2i+1 << 4
 * NaN inputs are outside the contract.
 * ------------------------------------------------------------------------- */
typedef enum bsfp4_cvt_mode {
  BSFP4_CVT_F32 = 0,
  BSFP4_CVT_BF16_E8M0 = 1,
  BSFP4_CVT_F32_E8M0 = 2
} bsfp4_cvt_mode;

BSFP4_API bsfp4_status bsfp4_e2m1_convert(int mode, const void* in, const uint8_t* scale_codes, int64_t pairs,
                                          uint8_t* codes, void* stream);

/* bsfp4_probe_mfma / bsfp4_probe_read: peak probes of the device, the rates
 * the kernels' roofline fractions are also reported against (beside the
 * published MI355X peaks).
 *   bsfp4_probe_mfma  kind 0 fp16 (v_mfma_f32_32x32x16_f16), 1 bf16, 2 fp8
 *                     E4M3 and 3 fp4 E2M1 (v_mfma_scale_f32_32x32x64_f8f6f4,
 *                     unit E8M0 scales), 4 / 5 fp16 / bf16 with operands of at
 *                     most 3 significant bits, 6 fp4 with random codes and 7
 *                     fp16 with random E2M1 x E4M3 products, both with
 *                     operands that change from one MFMA to the next (as in a
 *                     GEMM; the sustained rate of the power-limited part
 *                     depends on the operand data): every wave issues
 *                     `iters` x 8 independent MFMAs from registers, four
 *                     waves per SIMD; bsfp4_probe_mfma_flops(kind, iters) is
 *                     the launch's flop count (0 for invalid arguments), iters
 *                     in [1, 2^24] and a multiple of 4 for kinds 6 and 7
 *   bsfp4_probe_read  reads `bytes` (> 0, % 16 == 0) of device memory at
 *                     `buf` (16-byte aligned) once with 128-bit loads; writes
 *                     nothing
 * Both are asynchronous on `stream`; time them with events on that stream. */
BSFP4_API int64_t bsfp4_probe_mfma_flops(int kind, int iters);
BSFP4_API bsfp4_status bsfp4_probe_mfma(int kind, int iters, void* stream);
BSFP4_API bsfp4_status bsfp4_probe_read(const void* buf, int64_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BSFP4_H_ */

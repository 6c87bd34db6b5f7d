// C ABI of libbsfp4: argument validation, device check, dispatch.
//
// Every entry point validates all arguments before launching anything and
// reports the first violation through a status code plus a per-thread
// message.  Checks follow the pages' entry points (vLLM `sm103` branch
// comparison page: `scaled_fp4_quant_sm103a_impl` requires a row length
// divisible by 16 and bf16/fp16 input; `cutlass_scaled_fp4_mm_sm103a_impl`
// requires equal K, K % 32 == 0 and N % 32 == 0, contiguous scale tensors;
// "feat: sm100 cute_dsl w4a16 gemm" review: bf16 activations, aligned
// pointers, exact scale sizes) restated for this library's unpadded layouts.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/bsfp4.h"
#include "launchers.h"

namespace {

thread_local char g_err[512] = "";

bsfp4_status fail(bsfp4_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

bsfp4_status ok() {
  g_err[0] = '\0';
  return BSFP4_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// The MXFP4 kernels address an operand with 32-bit buffer offsets from its
// base (one expert's weights in the grouped form), so each must stay below
// 2^31 bytes.
constexpr int64_t kLim31 = (int64_t)1 << 31;

#define REQUIRE_PTR(p)                                                             \
  do {                                                                             \
    if ((p) == nullptr) return fail(BSFP4_ERR_INVALID_ARG, "%s is NULL", #p);      \
    if (!aligned((p), 16)) return fail(BSFP4_ERR_ALIGNMENT, "%s is not 16-byte aligned", #p); \
  } while (0)

#define REQUIRE_SCALAR_PTR(p)                                                      \
  do {                                                                             \
    if ((p) == nullptr) return fail(BSFP4_ERR_INVALID_ARG, "%s is NULL", #p);      \
    if (!aligned((p), 4)) return fail(BSFP4_ERR_ALIGNMENT, "%s is not 4-byte aligned", #p); \
  } while (0)

// The current device must be a gfx950; the answer is cached per device id.
bsfp4_status check_device() {
  static std::mutex mu;
  static int known[64] = {0};  // 0 unknown, 1 gfx950, 2 other
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0)
    return fail(BSFP4_ERR_DEVICE, "no HIP device: %s", hipGetErrorString(e));
  if (dev < 64) {
    std::lock_guard<std::mutex> lock(mu);
    if (known[dev] == 0) {
      hipDeviceProp_t prop;
      e = hipGetDeviceProperties(&prop, dev);
      if (e != hipSuccess) return fail(BSFP4_ERR_DEVICE, "hipGetDeviceProperties: %s", hipGetErrorString(e));
      known[dev] = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    }
    if (known[dev] == 1) return BSFP4_OK;
  }
  return fail(BSFP4_ERR_DEVICE, "device %d is not a gfx950 GPU", dev);
}

bsfp4_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(BSFP4_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

int bsfp4_version(void) { return 100; }

const char* bsfp4_status_string(int s) {
  switch (s) {
    case BSFP4_OK: return "ok";
    case BSFP4_ERR_INVALID_ARG: return "invalid argument";
    case BSFP4_ERR_SHAPE: return "unsupported shape";
    case BSFP4_ERR_ALIGNMENT: return "misaligned pointer";
    case BSFP4_ERR_WORKSPACE: return "workspace too small";
    case BSFP4_ERR_DEVICE: return "unsupported device";
    case BSFP4_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* bsfp4_last_error(void) { return g_err; }

// ------------------------------------------------------------------ global scale

size_t fp4_global_scale_workspace_size(int64_t numel) {
  if (numel <= 0) return 0;
  return sizeof(float) * (size_t)bsfp4::global_scale_parts(numel);
}

bsfp4_status fp4_global_scale(const uint16_t* x, int64_t numel, float* gs_out, void* ws,
                              size_t ws_bytes, void* stream) {
  if (numel <= 0) return fail(BSFP4_ERR_SHAPE, "numel must be > 0 (got %lld)", (long long)numel);
  REQUIRE_PTR(x);
  REQUIRE_SCALAR_PTR(gs_out);
  REQUIRE_SCALAR_PTR(ws);
  const size_t need = fp4_global_scale_workspace_size(numel);
  if (ws_bytes < need)
    return fail(BSFP4_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
  if (bsfp4_status s = check_device()) return s;
  return launched(bsfp4::launch_global_scale(x, numel, gs_out, static_cast<float*>(ws), as_stream(stream)),
                  "fp4_global_scale launch");
}

// ------------------------------------------------------------------ quantiser

bsfp4_status fp4_quantize(int fmt, const uint16_t* x, int64_t rows_in, int64_t K, const float* gs,
                          const int32_t* row_map, int64_t rows_out, uint8_t* q, uint8_t* sf,
                          void* stream) {
  if (fmt != BSFP4_NVFP4 && fmt != BSFP4_MXFP4) return fail(BSFP4_ERR_INVALID_ARG, "unknown format %d", fmt);
  if (rows_in < 0 || rows_out < 0 || K <= 0)
    return fail(BSFP4_ERR_SHAPE, "need rows >= 0 and K > 0 (rows_in=%lld rows_out=%lld K=%lld)",
                (long long)rows_in, (long long)rows_out, (long long)K);
  const int blk = fmt == BSFP4_NVFP4 ? 16 : 32;
  if (K % blk) return fail(BSFP4_ERR_SHAPE, "K=%lld is not a multiple of %d", (long long)K, blk);
  if (row_map == nullptr && rows_out != rows_in)
    return fail(BSFP4_ERR_SHAPE, "without row_map rows_out (%lld) must equal rows_in (%lld)",
                (long long)rows_out, (long long)rows_in);
  if (fmt == BSFP4_NVFP4) {
    REQUIRE_SCALAR_PTR(gs);
  } else if (gs != nullptr) {
    return fail(BSFP4_ERR_INVALID_ARG, "MXFP4 takes no global scale (gs must be NULL)");
  }
  if (rows_out == 0) return ok();
  if (rows_in > 0) REQUIRE_PTR(x);
  if (row_map != nullptr && !aligned(row_map, 4)) return fail(BSFP4_ERR_ALIGNMENT, "row_map is not 4-byte aligned");
  REQUIRE_PTR(q);
  if (sf == nullptr) return fail(BSFP4_ERR_INVALID_ARG, "sf is NULL");
  if (bsfp4_status s = check_device()) return s;
  return launched(bsfp4::launch_quantize(fmt, x, rows_in, K, gs, row_map, rows_out, q, sf, as_stream(stream)),
                  "fp4_quantize launch");
}

// ------------------------------------------------------------------ GEMM

size_t fp4_gemm_workspace_size(int fmt, int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N <= 0 || K <= 0) return 0;
  if (fmt == BSFP4_NVFP4) return bsfp4::nvfp4_gemm_workspace(M, N, K);
  return 0;
}

// Argument checks shared by fp4_gemm and fp4_gemm_noalloc (everything but the
// workspace).
static bsfp4_status check_gemm_args(int fmt, const uint8_t* A, const uint8_t* SFA, const uint8_t* B,
                                    const uint8_t* SFB, const float* alpha, const uint16_t* D, int64_t M, int64_t N,
                                    int64_t K) {
  if (fmt != BSFP4_NVFP4 && fmt != BSFP4_MXFP4) return fail(BSFP4_ERR_INVALID_ARG, "unknown format %d", fmt);
  if (M < 0 || N <= 0 || K <= 0)
    return fail(BSFP4_ERR_SHAPE, "need M >= 0, N > 0, K > 0 (M=%lld N=%lld K=%lld)", (long long)M,
                (long long)N, (long long)K);
  if (K % 32) return fail(BSFP4_ERR_SHAPE, "K=%lld is not a multiple of 32", (long long)K);
  if (N % 32) return fail(BSFP4_ERR_SHAPE, "N=%lld is not a multiple of 32", (long long)N);
  if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX)
    return fail(BSFP4_ERR_SHAPE, "dimensions must fit in 31 bits");
  if (fmt == BSFP4_MXFP4 && (M * (K / 2) >= kLim31 || N * (K / 2) >= kLim31))
    return fail(BSFP4_ERR_SHAPE, "MXFP4 operands must stay below 2^31 bytes (M*K/2=%lld, N*K/2=%lld)",
                (long long)(M * (K / 2)), (long long)(N * (K / 2)));
  if (M > 0) {
    REQUIRE_PTR(A);
    REQUIRE_PTR(SFA);
    REQUIRE_PTR(D);
  }
  REQUIRE_PTR(B);
  REQUIRE_PTR(SFB);
  if (alpha != nullptr && !aligned(alpha, 4)) return fail(BSFP4_ERR_ALIGNMENT, "alpha is not 4-byte aligned");
  return BSFP4_OK;
}

static bsfp4_status launch_gemm(int fmt, const uint8_t* A, const uint8_t* SFA, const uint8_t* B, const uint8_t* SFB,
                                const float* alpha, uint16_t* D, int64_t M, int64_t N, int64_t K, void* ws,
                                size_t ws_bytes, hipStream_t st) {
  if (fmt == BSFP4_NVFP4)
    return launched(bsfp4::launch_nvfp4_gemm(A, SFA, B, SFB, alpha, D, M, N, K, ws, ws_bytes, st), "fp4_gemm launch");
  return launched(bsfp4::launch_mxfp4_gemm(A, SFA, B, SFB, alpha, D, M, N, K, st), "fp4_gemm launch");
}

bsfp4_status fp4_gemm(int fmt, const uint8_t* A, const uint8_t* SFA, const uint8_t* B,
                      const uint8_t* SFB, const float* alpha, uint16_t* D, int64_t M, int64_t N,
                      int64_t K, void* ws, size_t ws_bytes, void* stream) {
  if (bsfp4_status s = check_gemm_args(fmt, A, SFA, B, SFB, alpha, D, M, N, K)) return s;
  const size_t need = fp4_gemm_workspace_size(fmt, M, N, K);
  if (need > 0) {
    if (ws == nullptr || ws_bytes < need)
      return fail(BSFP4_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws == nullptr ? 0 : ws_bytes, need);
    if (!aligned(ws, 16)) return fail(BSFP4_ERR_ALIGNMENT, "ws is not 16-byte aligned");
  }
  if (M == 0) return ok();
  if (bsfp4_status s = check_device()) return s;
  return launch_gemm(fmt, A, SFA, B, SFB, alpha, D, M, N, K, ws, ws_bytes, as_stream(stream));
}

size_t fp4_gemm_noalloc_max_workspace(void) { return bsfp4::kScratchBytes; }

bsfp4_status fp4_gemm_noalloc(int fmt, const uint8_t* A, const uint8_t* SFA, const uint8_t* B, const uint8_t* SFB,
                              const float* alpha, uint16_t* D, int64_t M, int64_t N, int64_t K, void* stream) {
  if (bsfp4_status s = check_gemm_args(fmt, A, SFA, B, SFB, alpha, D, M, N, K)) return s;
  const size_t need = fp4_gemm_workspace_size(fmt, M, N, K);
  if (need > bsfp4::kScratchBytes)
    return fail(BSFP4_ERR_WORKSPACE,
                "this shape needs %zu bytes of split-K partials, above the %zu-byte static scratch of "
                "fp4_gemm_noalloc (use fp4_gemm with a caller workspace)",
                need, bsfp4::kScratchBytes);
  if (M == 0) return ok();
  if (bsfp4_status s = check_device()) return s;
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t e = bsfp4::scratch_device_ptr(&ws);
    if (e != hipSuccess) return fail(BSFP4_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
  }
  return launch_gemm(fmt, A, SFA, B, SFB, alpha, D, M, N, K, ws, need > 0 ? bsfp4::kScratchBytes : 0,
                     as_stream(stream));
}

// ------------------------------------------------------------------ W4A16

size_t w4a16_gemm_workspace_size(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  if (bsfp4::w4a16_rows64_ok(M, N, K)) return bsfp4::w4a16_rows64_workspace(M, N, K);
  if (bsfp4::w4a16_tiled_ok(M, N, K)) return bsfp4::w4a16_tiled_workspace(M, N, K);
  // rows run in chunks of at most kSkinnyMaxM; the partials of one chunk are
  // reduced before the next chunk starts on the same stream
  const int64_t mc = M < bsfp4::kSkinnyMaxM ? M : bsfp4::kSkinnyMaxM;
  size_t need = bsfp4::skinny_workspace(mc, N, K, false);
  const int64_t tail = M % bsfp4::kSkinnyMaxM;
  if (M > bsfp4::kSkinnyMaxM && tail > 0) {
    const size_t t = bsfp4::skinny_workspace(tail, N, K, false);
    if (t > need) need = t;
  }
  return need;
}

bsfp4_status w4a16_gemm(const uint16_t* A, const uint8_t* B, const uint8_t* SFB, const float* alpha,
                        uint16_t* D, int64_t M, int64_t N, int64_t K, void* ws, size_t ws_bytes,
                        void* stream) {
  if (M < 0 || N <= 0 || K <= 0)
    return fail(BSFP4_ERR_SHAPE, "need M >= 0, N > 0, K > 0 (M=%lld N=%lld K=%lld)", (long long)M,
                (long long)N, (long long)K);
  if (K % 32) return fail(BSFP4_ERR_SHAPE, "K=%lld is not a multiple of 32", (long long)K);
  if (N % 32) return fail(BSFP4_ERR_SHAPE, "N=%lld is not a multiple of 32", (long long)N);
  if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX)
    return fail(BSFP4_ERR_SHAPE, "dimensions must fit in 31 bits");
  if (M > 0) {
    REQUIRE_PTR(A);
    REQUIRE_PTR(D);
  }
  REQUIRE_PTR(B);
  REQUIRE_PTR(SFB);
  if (alpha != nullptr && !aligned(alpha, 4)) return fail(BSFP4_ERR_ALIGNMENT, "alpha is not 4-byte aligned");
  const size_t need = w4a16_gemm_workspace_size(M, N, K);
  if (need > 0) {
    if (ws == nullptr || ws_bytes < need)
      return fail(BSFP4_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws == nullptr ? 0 : ws_bytes, need);
    if (!aligned(ws, 16)) return fail(BSFP4_ERR_ALIGNMENT, "ws is not 16-byte aligned");
  }
  if (M == 0) return ok();
  if (bsfp4_status s = check_device()) return s;
  if (bsfp4::w4a16_rows64_ok(M, N, K))
    return launched(bsfp4::launch_w4a16_rows64(A, B, SFB, alpha, D, M, N, K, static_cast<float*>(ws), ws_bytes,
                                               as_stream(stream)),
                    "w4a16_gemm launch");
  if (bsfp4::w4a16_tiled_ok(M, N, K))
    return launched(bsfp4::launch_w4a16_tiled(A, B, SFB, alpha, D, M, N, K, static_cast<float*>(ws), ws_bytes,
                                              as_stream(stream)),
                    "w4a16_gemm launch");
  // rows in chunks of kSkinnyMaxM (the weight stream is re-read once per chunk)
  for (int64_t m0 = 0; m0 < M; m0 += bsfp4::kSkinnyMaxM) {
    const int64_t mc = (M - m0 < bsfp4::kSkinnyMaxM) ? (M - m0) : bsfp4::kSkinnyMaxM;
    hipError_t e = bsfp4::launch_skinny_w4a16(A + m0 * K, B, SFB, alpha, D + m0 * N, mc, N, K,
                                              static_cast<float*>(ws), as_stream(stream));
    if (e != hipSuccess) return launched(e, "w4a16_gemm launch");
  }
  return ok();
}

// ------------------------------------------------------------------ E2M1 conversion

bsfp4_status bsfp4_e2m1_convert(int mode, const void* in, const uint8_t* scale_codes, int64_t pairs,
                                uint8_t* codes, void* stream) {
  if (mode != BSFP4_CVT_F32 && mode != BSFP4_CVT_BF16_E8M0 && mode != BSFP4_CVT_F32_E8M0)
    return fail(BSFP4_ERR_INVALID_ARG, "unknown conversion mode %d", mode);
  if (pairs < 0 || pairs % 4)
    return fail(BSFP4_ERR_SHAPE, "pairs must be >= 0 and a multiple of 4 (got %lld)", (long long)pairs);
  if (mode == BSFP4_CVT_F32) {
    if (scale_codes != nullptr) return fail(BSFP4_ERR_INVALID_ARG, "BSFP4_CVT_F32 takes no scale codes");
  }
  if (pairs == 0) return ok();
  REQUIRE_PTR(in);
  REQUIRE_PTR(codes);
  if (mode != BSFP4_CVT_F32) REQUIRE_PTR(scale_codes);
  if (bsfp4_status s = check_device()) return s;
  return launched(bsfp4::launch_e2m1_convert(mode, in, scale_codes, pairs, codes, as_stream(stream)),
                  "bsfp4_e2m1_convert launch");
}

// ------------------------------------------------------------------ peak probes

namespace {
int64_t mfma_flops(int kind) {
  return (kind == 2 || kind == 3 || kind == 6) ? 2LL * 32 * 32 * 64 : 2LL * 32 * 32 * 16;
}
// kinds 6 and 7 rotate four operand pairs: iters is a multiple of 4
bool probe_args_ok(int kind, int iters) {
  return kind >= 0 && kind <= 7 && iters > 0 && iters <= (1 << 24) && (kind < 6 || iters % 4 == 0);
}
}  // namespace

int64_t bsfp4_probe_mfma_flops(int kind, int iters) {
  if (!probe_args_ok(kind, iters)) return 0;
  // 8 MFMAs per iteration per wave, 4 waves per workgroup
  return bsfp4::probe_mfma_grid() * 4 * (int64_t)iters * 8 * mfma_flops(kind);
}

bsfp4_status bsfp4_probe_mfma(int kind, int iters, void* stream) {
  if (kind < 0 || kind > 7) return fail(BSFP4_ERR_INVALID_ARG, "unknown MFMA probe kind %d", kind);
  if (!probe_args_ok(kind, iters))
    return fail(BSFP4_ERR_SHAPE, "iters must be in [1, 2^24] and a multiple of 4 for kinds 6 and 7 (got %d)", iters);
  if (bsfp4_status s = check_device()) return s;
  return launched(bsfp4::launch_probe_mfma(kind, iters, as_stream(stream)), "bsfp4_probe_mfma launch");
}

bsfp4_status bsfp4_probe_read(const void* buf, int64_t bytes, void* stream) {
  if (bytes <= 0 || bytes % 16) return fail(BSFP4_ERR_SHAPE, "bytes must be a positive multiple of 16");
  REQUIRE_PTR(buf);
  if (bsfp4_status s = check_device()) return s;
  return launched(bsfp4::launch_probe_read(buf, bytes, as_stream(stream)), "bsfp4_probe_read launch");
}

// ------------------------------------------------------------------ scale layouts

size_t fp4_scales_swizzled_size(int64_t rows, int64_t kblocks) {
  if (rows < 0 || kblocks <= 0) return 0;
  return (size_t)((rows + 127) / 128 * 128) * (size_t)((kblocks + 3) / 4 * 4);
}

static bsfp4_status check_scale_layout(int layout, const void* a, const void* b, int64_t rows, int64_t kblocks,
                                       const void* swz) {
  if (layout != BSFP4_SF_128X4 && layout != BSFP4_SF_128X4_M8)
    return fail(BSFP4_ERR_INVALID_ARG, "unknown scale layout %d", layout);
  if (rows < 0 || kblocks <= 0)
    return fail(BSFP4_ERR_SHAPE, "need rows >= 0 and kblocks > 0 (rows=%lld kblocks=%lld)", (long long)rows,
                (long long)kblocks);
  if (rows > INT32_MAX || kblocks > INT32_MAX || fp4_scales_swizzled_size(rows, kblocks) >= ((size_t)1 << 31))
    return fail(BSFP4_ERR_SHAPE, "padded scale buffer must stay below 2^31 bytes");
  if (rows == 0) return ok();
  if (a == nullptr || b == nullptr) return fail(BSFP4_ERR_INVALID_ARG, "a scale pointer is NULL");
  if (!aligned(swz, 4)) return fail(BSFP4_ERR_ALIGNMENT, "the swizzled buffer is not 4-byte aligned");
  return ok();
}

bsfp4_status fp4_scales_swizzle(int layout, const uint8_t* sf, int64_t rows, int64_t kblocks, uint8_t* swz,
                                void* stream) {
  if (bsfp4_status s = check_scale_layout(layout, sf, swz, rows, kblocks, swz)) return s;
  if (rows == 0) return ok();
  if (bsfp4_status s = check_device()) return s;
  return launched(bsfp4::launch_scale_layout(layout, true, sf, swz, rows, kblocks, as_stream(stream)),
                  "fp4_scales_swizzle launch");
}

bsfp4_status fp4_scales_unswizzle(int layout, const uint8_t* swz, int64_t rows, int64_t kblocks, uint8_t* sf,
                                  void* stream) {
  if (bsfp4_status s = check_scale_layout(layout, swz, sf, rows, kblocks, swz)) return s;
  if (rows == 0) return ok();
  if (bsfp4_status s = check_device()) return s;
  return launched(bsfp4::launch_scale_layout(layout, false, swz, sf, rows, kblocks, as_stream(stream)),
                  "fp4_scales_unswizzle launch");
}

// ------------------------------------------------------------------ MoE

size_t fp4_moe_prep_workspace_size(int64_t T, int64_t topk, int64_t E) {
  (void)T;
  (void)topk;
  (void)E;
  return 0;
}

bsfp4_status fp4_moe_prep(const int32_t* topk_ids, int64_t T, int64_t topk, int64_t E,
                          int32_t* expert_offsets, int32_t* sorted_ids, int32_t* sorted_tokens, void* ws,
                          size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  if (T < 0 || topk <= 0 || E <= 0 || E > bsfp4::kMaxExperts)
    return fail(BSFP4_ERR_SHAPE, "need T >= 0, topk > 0, 0 < E <= %lld (T=%lld topk=%lld E=%lld)",
                (long long)bsfp4::kMaxExperts, (long long)T, (long long)topk, (long long)E);
  if (T * topk > INT32_MAX) return fail(BSFP4_ERR_SHAPE, "T*topk must fit in 31 bits");
  if (T > 0) {
    REQUIRE_PTR(topk_ids);
    if (sorted_ids == nullptr) return fail(BSFP4_ERR_INVALID_ARG, "sorted_ids is NULL");
    if (!aligned(sorted_ids, 4)) return fail(BSFP4_ERR_ALIGNMENT, "sorted_ids is not 4-byte aligned");
    if (sorted_tokens != nullptr && !aligned(sorted_tokens, 4))
      return fail(BSFP4_ERR_ALIGNMENT, "sorted_tokens is not 4-byte aligned");
  }
  if (expert_offsets == nullptr) return fail(BSFP4_ERR_INVALID_ARG, "expert_offsets is NULL");
  if (!aligned(expert_offsets, 4)) return fail(BSFP4_ERR_ALIGNMENT, "expert_offsets is not 4-byte aligned");
  if (bsfp4_status s = check_device()) return s;
  return launched(bsfp4::launch_moe_prep(topk_ids, T, topk, E, expert_offsets, sorted_ids, sorted_tokens,
                                         as_stream(stream)),
                  "fp4_moe_prep launch");
}

size_t mxfp4_moe_grouped_gemm_workspace_size(int64_t rows, int64_t E, int64_t N, int64_t K, int epilogue,
                                             int64_t num_tokens) {
  (void)E;
  (void)K;
  (void)num_tokens;
  if (epilogue == BSFP4_MOE_WEIGHTED_COMBINE && rows > 0 && N > 0)
    return (size_t)rows * (size_t)N * sizeof(float);
  return 0;
}

bsfp4_status mxfp4_moe_grouped_gemm(const uint8_t* Aq, const uint8_t* Asf, int64_t a_rows_total,
                                    const int32_t* a_row_index, const int32_t* expert_offsets, int64_t E,
                                    int64_t rows, const uint8_t* W, const uint8_t* Wsf, int64_t N, int64_t K,
                                    int epilogue, const bsfp4_moe_epilogue_args* ep, void* ws, size_t ws_bytes,
                                    void* stream) {
  if (epilogue != BSFP4_MOE_STORE_BF16 && epilogue != BSFP4_MOE_SILU_MUL_QUANT &&
      epilogue != BSFP4_MOE_WEIGHTED_COMBINE)
    return fail(BSFP4_ERR_INVALID_ARG, "unknown epilogue %d", epilogue);
  if (ep == nullptr) return fail(BSFP4_ERR_INVALID_ARG, "ep is NULL");
  if (rows < 0 || a_rows_total < 0 || E <= 0 || E > bsfp4::kMaxExperts || N <= 0 || K <= 0)
    return fail(BSFP4_ERR_SHAPE, "need rows >= 0, a_rows_total >= 0, 0 < E <= %lld, N > 0, K > 0",
                (long long)bsfp4::kMaxExperts);
  if (a_row_index == nullptr && a_rows_total != rows)
    return fail(BSFP4_ERR_SHAPE, "without a_row_index, a_rows_total (%lld) must equal rows (%lld)",
                (long long)a_rows_total, (long long)rows);
  if (K % 32) return fail(BSFP4_ERR_SHAPE, "K=%lld is not a multiple of 32", (long long)K);
  if (N % 32) return fail(BSFP4_ERR_SHAPE, "N=%lld is not a multiple of 32", (long long)N);
  if (epilogue == BSFP4_MOE_SILU_MUL_QUANT && N % 64)
    return fail(BSFP4_ERR_SHAPE, "SILU_MUL_QUANT needs N %% 64 == 0 (got N=%lld)", (long long)N);
  if (rows > INT32_MAX || a_rows_total > INT32_MAX || N > INT32_MAX || K > INT32_MAX)
    return fail(BSFP4_ERR_SHAPE, "dimensions must fit in 31 bits");
  if (a_rows_total * (K / 2) >= kLim31 || N * (K / 2) >= kLim31)
    return fail(BSFP4_ERR_SHAPE, "Aq (a_rows_total*K/2=%lld) and one expert's W (N*K/2=%lld) must stay below 2^31 bytes",
                (long long)(a_rows_total * (K / 2)), (long long)(N * (K / 2)));
  REQUIRE_PTR(W);
  REQUIRE_PTR(Wsf);
  REQUIRE_PTR(expert_offsets);
  if (a_row_index != nullptr && !aligned(a_row_index, 4))
    return fail(BSFP4_ERR_ALIGNMENT, "a_row_index is not 4-byte aligned");
  if (rows > 0) {
    REQUIRE_PTR(Aq);
    REQUIRE_PTR(Asf);
    if (epilogue == BSFP4_MOE_STORE_BF16) {
      if (ep->out == nullptr) return fail(BSFP4_ERR_INVALID_ARG, "ep.out is NULL");
      if (!aligned(ep->out, 16)) return fail(BSFP4_ERR_ALIGNMENT, "ep.out is not 16-byte aligned");
    } else if (epilogue == BSFP4_MOE_SILU_MUL_QUANT) {
      if (ep->out_q == nullptr || ep->out_sf == nullptr) return fail(BSFP4_ERR_INVALID_ARG, "ep.out_q/out_sf is NULL");
      if (!aligned(ep->out_q, 16)) return fail(BSFP4_ERR_ALIGNMENT, "ep.out_q is not 16-byte aligned");
    }
  }
  const int64_t T = ep->num_tokens;
  if (epilogue == BSFP4_MOE_WEIGHTED_COMBINE) {
    if (T <= 0 || ep->topk <= 0 || T * ep->topk != rows)
      return fail(BSFP4_ERR_SHAPE, "WEIGHTED_COMBINE needs num_tokens*topk == rows (T=%lld topk=%lld rows=%lld)",
                  (long long)T, (long long)ep->topk, (long long)rows);
    if (ep->out == nullptr || ep->sorted_ids == nullptr || ep->topk_weights == nullptr)
      return fail(BSFP4_ERR_INVALID_ARG, "ep.out / sorted_ids / topk_weights is NULL");
    if (!aligned(ep->out, 16)) return fail(BSFP4_ERR_ALIGNMENT, "ep.out is not 16-byte aligned");
    const size_t need = mxfp4_moe_grouped_gemm_workspace_size(rows, E, N, K, epilogue, T);
    if (ws == nullptr || ws_bytes < need)
      return fail(BSFP4_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws == nullptr ? 0 : ws_bytes, need);
    if (!aligned(ws, 16)) return fail(BSFP4_ERR_ALIGNMENT, "ws is not 16-byte aligned");
  }
  if (rows == 0) return ok();
  if (bsfp4_status s = check_device()) return s;
  const hipStream_t st = as_stream(stream);
  if (epilogue == BSFP4_MOE_WEIGHTED_COMBINE) {
    float* y = static_cast<float*>(ws);
    hipError_t e = bsfp4::launch_mxfp4_grouped(Aq, Asf, a_row_index, a_rows_total, expert_offsets, E, rows, W, Wsf,
                                               N, K, bsfp4::kEpiCombine, nullptr, nullptr, nullptr, ep->sorted_ids, y,
                                               st);
    if (e == hipSuccess)
      e = bsfp4::launch_topk_sum(y, ep->topk_weights, static_cast<uint16_t*>(ep->out), T, ep->topk, N, st);
    return launched(e, "mxfp4_moe_grouped_gemm launch");
  }
  return launched(bsfp4::launch_mxfp4_grouped(Aq, Asf, a_row_index, a_rows_total, expert_offsets, E, rows, W, Wsf,
                                              N, K,
                                              epilogue == BSFP4_MOE_STORE_BF16 ? bsfp4::kEpiStore : bsfp4::kEpiSilu,
                                              static_cast<uint16_t*>(ep->out), ep->out_q, ep->out_sf, nullptr,
                                              nullptr, st),
                  "mxfp4_moe_grouped_gemm launch");
}

// ------------------------------------------------------------------ quantise + GEMM

namespace {
int64_t round16(int64_t b) { return (b + 15) / 16 * 16; }
}  // namespace

size_t nvfp4_quantize_gemm_workspace_size(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0 || K % 32 || N % 32) return 0;
  if (bsfp4::nvfp4_fused_quant_gemm_ok(M, N, K)) return 0;
  return (size_t)(round16(M * (K / 2)) + round16(M * (K / 16))) + bsfp4::nvfp4_gemm_workspace(M, N, K);
}

bsfp4_status nvfp4_quantize_gemm(const uint16_t* x, const float* gs, const uint8_t* B, const uint8_t* SFB,
                                 const float* alpha, uint16_t* D, int64_t M, int64_t N, int64_t K, void* ws,
                                 size_t ws_bytes, void* stream) {
  if (M < 0 || N <= 0 || K <= 0)
    return fail(BSFP4_ERR_SHAPE, "need M >= 0, N > 0, K > 0 (M=%lld N=%lld K=%lld)", (long long)M, (long long)N,
                (long long)K);
  if (K % 32) return fail(BSFP4_ERR_SHAPE, "K=%lld is not a multiple of 32", (long long)K);
  if (N % 32) return fail(BSFP4_ERR_SHAPE, "N=%lld is not a multiple of 32", (long long)N);
  if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return fail(BSFP4_ERR_SHAPE, "dimensions must fit in 31 bits");
  REQUIRE_SCALAR_PTR(gs);
  REQUIRE_PTR(B);
  REQUIRE_PTR(SFB);
  if (alpha != nullptr && !aligned(alpha, 4)) return fail(BSFP4_ERR_ALIGNMENT, "alpha is not 4-byte aligned");
  if (M > 0) {
    REQUIRE_PTR(x);
    REQUIRE_PTR(D);
  }
  const size_t need = nvfp4_quantize_gemm_workspace_size(M, N, K);
  if (need > 0) {
    if (ws == nullptr || ws_bytes < need)
      return fail(BSFP4_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws == nullptr ? 0 : ws_bytes, need);
    if (!aligned(ws, 16)) return fail(BSFP4_ERR_ALIGNMENT, "ws is not 16-byte aligned");
  }
  if (M == 0) return ok();
  if (bsfp4_status s = check_device()) return s;
  const hipStream_t st = as_stream(stream);
  if (need == 0)
    return launched(bsfp4::launch_nvfp4_fused_quant_gemm(x, gs, B, SFB, alpha, D, M, N, K, st),
                    "nvfp4_quantize_gemm launch");
  uint8_t* q = static_cast<uint8_t*>(ws);
  uint8_t* sf = q + round16(M * (K / 2));
  uint8_t* gws = sf + round16(M * (K / 16));
  const size_t gws_bytes = ws_bytes - (size_t)(gws - q);
  hipError_t e = bsfp4::launch_quantize(0, x, M, K, gs, nullptr, M, q, sf, st);
  if (e == hipSuccess) e = bsfp4::launch_nvfp4_gemm(q, sf, B, SFB, alpha, D, M, N, K, gws, gws_bytes, st);
  return launched(e, "nvfp4_quantize_gemm launch");
}

// ------------------------------------------------------------------ NVFP4 MoE

bsfp4_status nvfp4_experts_quantize(const uint16_t* x, int64_t rows_in, int64_t K, const int32_t* row_map,
                                    const int32_t* expert_offsets, int64_t E, const float* gs_experts,
                                    int64_t rows_out, uint8_t* q, uint8_t* sf, void* stream) {
  if (rows_in < 0 || rows_out < 0 || K <= 0)
    return fail(BSFP4_ERR_SHAPE, "need rows >= 0 and K > 0 (rows_in=%lld rows_out=%lld K=%lld)",
                (long long)rows_in, (long long)rows_out, (long long)K);
  if (K % 16) return fail(BSFP4_ERR_SHAPE, "K=%lld is not a multiple of 16", (long long)K);
  if (E <= 0 || E > bsfp4::kMaxExperts)
    return fail(BSFP4_ERR_SHAPE, "need 0 < E <= %lld (E=%lld)", (long long)bsfp4::kMaxExperts, (long long)E);
  if (row_map == nullptr && rows_out != rows_in)
    return fail(BSFP4_ERR_SHAPE, "without row_map rows_out (%lld) must equal rows_in (%lld)",
                (long long)rows_out, (long long)rows_in);
  REQUIRE_PTR(expert_offsets);
  REQUIRE_PTR(gs_experts);
  if (!aligned(expert_offsets, 4) || !aligned(gs_experts, 4))
    return fail(BSFP4_ERR_ALIGNMENT, "expert_offsets / gs_experts are not 4-byte aligned");
  if (rows_out == 0) return ok();
  if (rows_in > 0) REQUIRE_PTR(x);
  if (row_map != nullptr && !aligned(row_map, 4)) return fail(BSFP4_ERR_ALIGNMENT, "row_map is not 4-byte aligned");
  REQUIRE_PTR(q);
  if (sf == nullptr) return fail(BSFP4_ERR_INVALID_ARG, "sf is NULL");
  if (bsfp4_status s = check_device()) return s;
  return launched(bsfp4::launch_nvfp4_experts_quant(x, rows_in, K, row_map, expert_offsets, E, gs_experts, rows_out,
                                                    q, sf, as_stream(stream)),
                  "nvfp4_experts_quantize launch");
}

size_t nvfp4_moe_grouped_gemm_workspace_size(int64_t rows, int64_t E, int64_t N, int64_t K, int epilogue,
                                             int64_t num_tokens) {
  (void)E;
  (void)K;
  (void)num_tokens;
  if (epilogue == BSFP4_MOE_WEIGHTED_COMBINE && rows > 0 && N > 0)
    return (size_t)rows * (size_t)N * sizeof(float);
  return 0;
}

bsfp4_status nvfp4_moe_grouped_gemm(const uint8_t* Aq, const uint8_t* Asf, const int32_t* expert_offsets,
                                    int64_t E, int64_t rows, const uint8_t* W, const uint8_t* Wsf,
                                    const float* alpha_experts, int64_t N, int64_t K, int epilogue,
                                    const bsfp4_moe_epilogue_args* ep, void* ws, size_t ws_bytes, void* stream) {
  if (epilogue != BSFP4_MOE_STORE_BF16 && epilogue != BSFP4_MOE_SILU_MUL_QUANT &&
      epilogue != BSFP4_MOE_WEIGHTED_COMBINE)
    return fail(BSFP4_ERR_INVALID_ARG, "unknown epilogue %d", epilogue);
  if (ep == nullptr) return fail(BSFP4_ERR_INVALID_ARG, "ep is NULL");
  if (rows < 0 || E <= 0 || E > bsfp4::kMaxExperts || N <= 0 || K <= 0)
    return fail(BSFP4_ERR_SHAPE, "need rows >= 0, 0 < E <= %lld, N > 0, K > 0", (long long)bsfp4::kMaxExperts);
  if (K % 32) return fail(BSFP4_ERR_SHAPE, "K=%lld is not a multiple of 32", (long long)K);
  if (N % 32) return fail(BSFP4_ERR_SHAPE, "N=%lld is not a multiple of 32", (long long)N);
  if (epilogue == BSFP4_MOE_SILU_MUL_QUANT && N % 64)
    return fail(BSFP4_ERR_SHAPE, "SILU_MUL_QUANT needs N %% 64 == 0 (got N=%lld)", (long long)N);
  if (rows > INT32_MAX || N * (K / 2) >= ((int64_t)1 << 31))
    return fail(BSFP4_ERR_SHAPE, "rows must fit in 31 bits and one expert's N*K/2 bytes below 2^31");
  REQUIRE_PTR(W);
  REQUIRE_PTR(Wsf);
  REQUIRE_PTR(expert_offsets);
  if (!aligned(expert_offsets, 4)) return fail(BSFP4_ERR_ALIGNMENT, "expert_offsets is not 4-byte aligned");
  if (alpha_experts != nullptr && !aligned(alpha_experts, 4))
    return fail(BSFP4_ERR_ALIGNMENT, "alpha_experts is not 4-byte aligned");
  if (rows > 0) {
    REQUIRE_PTR(Aq);
    REQUIRE_PTR(Asf);
    if (epilogue == BSFP4_MOE_STORE_BF16) {
      if (ep->out == nullptr) return fail(BSFP4_ERR_INVALID_ARG, "ep.out is NULL");
      if (!aligned(ep->out, 16)) return fail(BSFP4_ERR_ALIGNMENT, "ep.out is not 16-byte aligned");
    } else if (epilogue == BSFP4_MOE_SILU_MUL_QUANT) {
      if (ep->out_q == nullptr || ep->out_sf == nullptr || ep->out_gs == nullptr)
        return fail(BSFP4_ERR_INVALID_ARG, "ep.out_q / out_sf / out_gs is NULL");
      if (!aligned(ep->out_q, 16)) return fail(BSFP4_ERR_ALIGNMENT, "ep.out_q is not 16-byte aligned");
      if (!aligned(ep->out_sf, 2)) return fail(BSFP4_ERR_ALIGNMENT, "ep.out_sf is not 2-byte aligned");
      if (!aligned(ep->out_gs, 4)) return fail(BSFP4_ERR_ALIGNMENT, "ep.out_gs is not 4-byte aligned");
    }
  }
  const int64_t T = ep->num_tokens;
  if (epilogue == BSFP4_MOE_WEIGHTED_COMBINE) {
    if (T <= 0 || ep->topk <= 0 || T * ep->topk != rows)
      return fail(BSFP4_ERR_SHAPE, "WEIGHTED_COMBINE needs num_tokens*topk == rows (T=%lld topk=%lld rows=%lld)",
                  (long long)T, (long long)ep->topk, (long long)rows);
    if (ep->out == nullptr || ep->sorted_ids == nullptr || ep->topk_weights == nullptr)
      return fail(BSFP4_ERR_INVALID_ARG, "ep.out / sorted_ids / topk_weights is NULL");
    if (!aligned(ep->out, 16)) return fail(BSFP4_ERR_ALIGNMENT, "ep.out is not 16-byte aligned");
    const size_t need = nvfp4_moe_grouped_gemm_workspace_size(rows, E, N, K, epilogue, T);
    if (ws == nullptr || ws_bytes < need)
      return fail(BSFP4_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws == nullptr ? 0 : ws_bytes, need);
    if (!aligned(ws, 16)) return fail(BSFP4_ERR_ALIGNMENT, "ws is not 16-byte aligned");
  }
  if (rows == 0) return ok();
  if (bsfp4_status s = check_device()) return s;
  const hipStream_t st = as_stream(stream);
  if (epilogue == BSFP4_MOE_WEIGHTED_COMBINE) {
    float* y = static_cast<float*>(ws);
    hipError_t e = bsfp4::launch_nvfp4_grouped(Aq, Asf, expert_offsets, E, rows, W, Wsf, alpha_experts, N, K,
                                               bsfp4::kEpiCombine, nullptr, nullptr, nullptr, nullptr,
                                               ep->sorted_ids, y, st);
    if (e == hipSuccess)
      e = bsfp4::launch_topk_sum(y, ep->topk_weights, static_cast<uint16_t*>(ep->out), T, ep->topk, N, st);
    return launched(e, "nvfp4_moe_grouped_gemm launch");
  }
  return launched(bsfp4::launch_nvfp4_grouped(Aq, Asf, expert_offsets, E, rows, W, Wsf, alpha_experts, N, K,
                                              epilogue == BSFP4_MOE_STORE_BF16 ? bsfp4::kEpiStore : bsfp4::kEpiSilu,
                                              static_cast<uint16_t*>(ep->out), ep->out_q, ep->out_sf, ep->out_gs,
                                              nullptr, nullptr, st),
                  "nvfp4_moe_grouped_gemm launch");
}

}  // extern "C"

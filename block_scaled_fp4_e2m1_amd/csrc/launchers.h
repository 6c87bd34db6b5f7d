// Host-side launchers of the gfx950 kernels (internal to libbsfp4).  Each
// assumes its arguments were validated by the C ABI layer and launches on
// the given stream; it returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bsfp4 {

constexpr int64_t kQuantMaxGrid = 4096;
constexpr int64_t kAmaxMaxParts = 1024;

hipError_t launch_quantize(int fmt, const uint16_t* x, int64_t rows_in, int64_t K, const float* gs,
                           const int32_t* row_map, int64_t rows_out, uint8_t* q, uint8_t* sf,
                           hipStream_t stream);

int global_scale_parts(int64_t numel);
hipError_t launch_global_scale(const uint16_t* x, int64_t numel, float* gs, float* partial,
                               hipStream_t stream);

hipError_t launch_nvfp4_gemm(const uint8_t* A, const uint8_t* SFA, const uint8_t* B, const uint8_t* SFB,
                             const float* alpha, uint16_t* D, int64_t M, int64_t N, int64_t K,
                             void* ws, size_t ws_bytes, hipStream_t stream);
size_t nvfp4_gemm_workspace(int64_t M, int64_t N, int64_t K);

}  // namespace bsfp4

// Block-scale layout interchange: row-major [rows, kblocks] bytes (the layout
// of every scale tensor in this library) <-> the padded, swizzled layouts the
// pages' block-scaled GEMMs consume (vLLM `sm103` branch comparison page,
// `nvfp4_quant_kernels.cu` and `nvfp4_scaled_mm_entry.cu`):
//   * padded shape [round_up(rows, 128), round_up(kblocks, 4)];
//   * 512-byte tiles of 128 rows x 4 scale columns, tile (row tile, column
//     tile) at (row_tile * column_tiles + column_tile) * 512;
//   * inside a tile the 4 columns of local row r are 4 consecutive bytes at
//       layout 0 (the SM100 form):  (r % 32) * 16 + (r / 32) * 4
//       layout 1 (the SM103 form):  (r / 16) * 16 + ((r / 4) % 4) * 128 + (r % 4) * 4.
// One thread per such 4-byte group: the swizzled side moves as one dword
// (coalesced), the row-major side byte by byte (its rows are kblocks bytes, not
// dword aligned in general).  Padding is written as zeros.
#include "device_common.h"
#include "launchers.h"

namespace bsfp4 {
namespace {

// dword index d inside a tile -> local row
template <int LAYOUT>
__device__ __forceinline__ int local_row(int d) {
  if constexpr (LAYOUT == 0) return (d >> 2) + 32 * (d & 3);  // d = (r % 32) * 4 + r / 32
  return (d & 3) + 4 * (d >> 5) + 16 * ((d >> 2) & 7);         // d = (r/16)*4 + ((r/4)%4)*32 + r%4
}

template <int LAYOUT, bool TO_SWIZZLED>
__global__ void __launch_bounds__(256)
    scale_layout(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, int rows, int kblocks, int col_tiles,
                 int64_t dwords) {
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < dwords; t += (int64_t)gridDim.x * 256) {
    const int64_t tile = t >> 7;
    const int m = (int)(tile / col_tiles) * 128 + local_row<LAYOUT>((int)(t & 127));
    const int k0 = (int)(tile % col_tiles) * 4;
    const int64_t row = (int64_t)m * kblocks;
    if constexpr (TO_SWIZZLED) {
      uint32_t v = 0;
      if (m < rows) {
#pragma unroll
        for (int c = 0; c < 4; c++)
          if (k0 + c < kblocks) v |= (uint32_t)src[row + k0 + c] << (8 * c);
      }
      reinterpret_cast<uint32_t*>(dst)[t] = v;
    } else {
      if (m >= rows) continue;
      const uint32_t v = reinterpret_cast<const uint32_t*>(src)[t];
#pragma unroll
      for (int c = 0; c < 4; c++)
        if (k0 + c < kblocks) dst[row + k0 + c] = (uint8_t)(v >> (8 * c));
    }
  }
}

template <int LAYOUT>
hipError_t launch_layout(bool to_swizzled, const uint8_t* src, uint8_t* dst, int64_t rows, int64_t kblocks,
                         hipStream_t stream) {
  const int64_t col_tiles = (kblocks + 3) / 4, row_tiles = (rows + 127) / 128;
  const int64_t dwords = row_tiles * col_tiles * 128;
  const int64_t blocks = (dwords + 255) / 256;
  const unsigned grid = (unsigned)(blocks < 4096 ? blocks : 4096);
  if (to_swizzled)
    scale_layout<LAYOUT, true><<<grid, 256, 0, stream>>>(src, dst, (int)rows, (int)kblocks, (int)col_tiles, dwords);
  else
    scale_layout<LAYOUT, false><<<grid, 256, 0, stream>>>(src, dst, (int)rows, (int)kblocks, (int)col_tiles, dwords);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_scale_layout(int layout, bool to_swizzled, const uint8_t* src, uint8_t* dst, int64_t rows,
                               int64_t kblocks, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  return layout == 0 ? launch_layout<0>(to_swizzled, src, dst, rows, kblocks, stream)
                     : launch_layout<1>(to_swizzled, src, dst, rows, kblocks, stream);
}

}  // namespace bsfp4

"""Block-scale layout interchange: canonical row-major <-> 128x4 swizzled (CPU oracle).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The library keeps block scales row-major, one byte per block: [rows, K/16]
(NVFP4) or [rows, K/32] (MXFP4).  The pages' kernels take them padded and
swizzled instead; this module writes that layout out from the pages' text:

  * padded shape [round_up(rows, 128), round_up(kblocks, 4)] bytes (vLLM
    `sm103` branch comparison page, `nvfp4_scaled_mm_entry.cu`, the shape
    checks of the SM103 scaled-mm entry);
  * the buffer is a run of 512-byte tiles of 128 rows x 4 scale columns, tile
    (row tile mt, column tile kt) starting at byte (mt * column_tiles + kt) * 512
    (same page, `nvfp4_quant_kernels.cu`, the SM103 scale-offset helper);
  * inside a tile, the byte of local row r (0..127) and local column c (0..3) is
      layout "128x4" (the SM100 form):  (r % 32) * 16 + (r // 32) * 4 + c
      layout "128x4_m8" (the SM103 form): (r // 16) * 16 + ((r // 4) % 4) * 128
                                          + (r % 4) * 4 + c
    (same page, the comment block of the SM100 <-> SM103 conversion kernel and
    the SM103 offset helper);
  * bytes of the padding (rows >= rows, columns >= kblocks) are zero.

Reading taken: the SM103 atom's printed CuTe shape/stride pair lists its row
modes in an order that does not match the decomposition the same helper
computes (r = r4b + 4 r4a + 16 r8); the explicit offset formula above is
followed.
"""
from __future__ import annotations

import numpy as np

LAYOUTS = ("128x4", "128x4_m8")
TILE_ROWS, TILE_COLS, TILE_BYTES = 128, 4, 512


def round_up(x: int, y: int) -> int:
    return (x + y - 1) // y * y


def swizzled_shape(rows: int, kblocks: int) -> tuple[int, int]:
    """Padded shape of the swizzled buffer, in bytes: (rows', kblocks')."""
    return round_up(rows, TILE_ROWS), round_up(kblocks, TILE_COLS)


def tile_offset(layout: str, r: int, c: int) -> int:
    """Byte offset of local (row r, column c) inside one 512-byte tile."""
    if not (0 <= r < TILE_ROWS and 0 <= c < TILE_COLS):
        raise ValueError("local index out of the tile")
    if layout == "128x4":
        return (r % 32) * 16 + (r // 32) * 4 + c
    if layout == "128x4_m8":
        return (r // 16) * 16 + ((r // 4) % 4) * 128 + (r % 4) * 4 + c
    raise ValueError(f"unknown layout {layout!r}")


def offset(layout: str, m: int, k: int, kblocks: int) -> int:
    """Byte offset of scale (row m, block k) in the swizzled buffer."""
    col_tiles = round_up(kblocks, TILE_COLS) // TILE_COLS
    tile = (m // TILE_ROWS) * col_tiles + k // TILE_COLS
    return tile * TILE_BYTES + tile_offset(layout, m % TILE_ROWS, k % TILE_COLS)


def swizzle(sf: np.ndarray, layout: str) -> np.ndarray:
    """Canonical [rows, kblocks] uint8 -> padded swizzled bytes, shape (rows', kblocks')."""
    sf = np.asarray(sf, dtype=np.uint8)
    rows, kblocks = sf.shape
    R, C = swizzled_shape(rows, kblocks)
    out = np.zeros(R * C, dtype=np.uint8)
    for m in range(rows):
        for k in range(kblocks):
            out[offset(layout, m, k, kblocks)] = sf[m, k]
    return out.reshape(R, C)


def unswizzle(buf: np.ndarray, rows: int, kblocks: int, layout: str) -> np.ndarray:
    """Padded swizzled bytes -> canonical [rows, kblocks] uint8 (the padding is dropped)."""
    flat = np.asarray(buf, dtype=np.uint8).reshape(-1)
    R, C = swizzled_shape(rows, kblocks)
    if flat.size != R * C:
        raise ValueError("buffer size does not match the padded shape")
    sf = np.empty((rows, kblocks), dtype=np.uint8)
    for m in range(rows):
        for k in range(kblocks):
            sf[m, k] = flat[offset(layout, m, k, kblocks)]
    return sf

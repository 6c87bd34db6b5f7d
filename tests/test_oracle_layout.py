"""Pins of the scale-layout oracle (oracle/layout.py) against facts fixed
outside its per-element formula:
  * hand-worked byte offsets (tests/golden/layout_examples.json);
  * the layouts are permutations of the padded buffer, with zero padding;
  * the 128x4 buffer seen as the 6-D strided view described on the FlashInfer
    trace page -- physical (row tile, column tile, 32, 4, 4) read in logical
    order (outer row, inner row, row tile, inner column, column tile) -- is the
    canonical matrix: element [o, i, mt, ic, kt] = sf[mt*128 + 32*i + o, 4*kt + ic]
    (done with numpy reshapes and transposes, not the offset formula);
  * the 128x4_m8 tile seen as physical (r4a, r8, r4b, column) = (4, 8, 4, 4) is
    the tile's rows in order r = r4b + 4*r4a + 16*r8 (again by reshape);
  * unswizzle inverts swizzle.
"""
import json
import os

import numpy as np
import pytest

from oracle import layout as L
from block_scaled_fp4_e2m1_amd import synth

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "layout_examples.json")))


@pytest.mark.parametrize("case", GOLDEN["offsets"], ids=lambda c: f"{c['layout']}-m{c['m']}-k{c['k']}")
def test_hand_worked_offsets(case):
    assert L.offset(case["layout"], case["m"], case["k"], case["kblocks"]) == case["offset"]


@pytest.mark.parametrize("layout", L.LAYOUTS)
@pytest.mark.parametrize("rows,kblocks", [(1, 1), (128, 4), (129, 5), (300, 13), (256, 8)])
def test_permutation_and_zero_padding(layout, rows, kblocks):
    R, C = L.swizzled_shape(rows, kblocks)
    offs = [L.offset(layout, m, k, C) for m in range(R) for k in range(C)]
    assert sorted(offs) == list(range(R * C))
    sf = synth.random_bytes(7, (rows, kblocks))
    buf = L.swizzle(sf, layout).reshape(-1)
    used = {L.offset(layout, m, k, kblocks) for m in range(rows) for k in range(kblocks)}
    pad = np.array(sorted(set(range(R * C)) - used), dtype=np.int64)
    assert np.all(buf[pad] == 0) if pad.size else True


@pytest.mark.parametrize("rows,kblocks", [(128, 4), (256, 12), (300, 7)])
def test_128x4_is_the_six_dim_view(rows, kblocks):
    sf = synth.random_bytes(11, (rows, kblocks))
    R, C = L.swizzled_shape(rows, kblocks)
    buf = L.swizzle(sf, "128x4")
    phys = buf.reshape(R // 128, C // 4, 32, 4, 4)  # (row tile, column tile, outer, inner, column)
    logical = phys.transpose(2, 3, 0, 4, 1)         # (outer, inner, row tile, inner column, column tile)
    padded = np.zeros((R, C), np.uint8)
    padded[:rows, :kblocks] = sf
    want = padded.reshape(R // 128, 4, 32, C // 4, 4).transpose(2, 1, 0, 4, 3)
    assert np.array_equal(logical, want)


@pytest.mark.parametrize("rows,kblocks", [(128, 4), (384, 8), (129, 3)])
def test_128x4_m8_tile_reshape(rows, kblocks):
    sf = synth.random_bytes(12, (rows, kblocks))
    R, C = L.swizzled_shape(rows, kblocks)
    buf = L.swizzle(sf, "128x4_m8").reshape(R // 128, C // 4, 4, 8, 4, 4)  # (mt, kt, r4a, r8, r4b, c)
    rowsorted = buf.transpose(0, 3, 2, 4, 1, 5).reshape(R, C)                # rows r8*16 + r4a*4 + r4b
    padded = np.zeros((R, C), np.uint8)
    padded[:rows, :kblocks] = sf
    assert np.array_equal(rowsorted, padded)


@pytest.mark.parametrize("layout", L.LAYOUTS)
def test_round_trip(layout):
    sf = synth.random_bytes(13, (200, 30))
    assert np.array_equal(L.unswizzle(L.swizzle(sf, layout), 200, 30, layout), sf)

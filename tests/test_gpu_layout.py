"""GPU parity: block-scale layout interchange (fp4_scales_swizzle /
fp4_scales_unswizzle) against the oracle, byte for byte, for both tile forms,
ragged row and column counts, and the scales fp4_quantize writes for the
4096 x 7168 workload."""
import numpy as np
import pytest
import torch

import block_scaled_fp4_e2m1_amd as bs
from block_scaled_fp4_e2m1_amd import synth
from oracle import layout as OL
from gpu_helpers import dev_u8

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("layout", ["128x4", "128x4_m8"])
@pytest.mark.parametrize("rows,kblocks", [(1, 1), (5, 3), (128, 4), (129, 5), (300, 13), (256, 448), (1000, 64)])
def test_scales_swizzle_matches_oracle(layout, rows, kblocks):
    sf = synth.random_bytes(rows * 7 + kblocks, (rows, kblocks))
    swz = bs.scales_swizzle(dev_u8(sf), layout)
    torch.cuda.synchronize()
    want = OL.swizzle(sf, layout)
    assert swz.shape == want.shape
    assert np.array_equal(swz.cpu().numpy(), want)
    back = bs.scales_unswizzle(swz, rows, kblocks, layout)
    torch.cuda.synchronize()
    assert np.array_equal(back.cpu().numpy(), sf)


@pytest.mark.parametrize("layout", ["128x4", "128x4_m8"])
def test_unswizzle_of_oracle_buffer(layout):
    """A buffer laid out by the oracle (padding included) reads back as the canonical matrix."""
    rows, kblocks = 333, 29
    sf = synth.random_bytes(5, (rows, kblocks))
    buf = OL.swizzle(sf, layout)
    got = bs.scales_unswizzle(dev_u8(buf), rows, kblocks, layout)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), sf)


def test_workload_scales_round_trip():
    """The E4M3 scales of a quantised 4096 x 7168 weight, swizzled and back."""
    w = synth.bf16_normal(3, (4096, 7168), 0.02)
    x = torch.from_numpy(w.view(np.int16)).cuda().view(torch.bfloat16)
    _, sf = bs.quantize(x, "nvfp4", gs=bs.global_scale(x))
    for layout in ("128x4", "128x4_m8"):
        swz = bs.scales_swizzle(sf, layout)
        back = bs.scales_unswizzle(swz, 4096, 448, layout)
        torch.cuda.synchronize()
        assert torch.equal(back, sf)
    h = sf.cpu().numpy()
    want = OL.swizzle(h[:256], "128x4_m8")  # first two row tiles against the oracle
    got = bs.scales_swizzle(sf[:256].contiguous(), "128x4_m8").cpu().numpy()
    assert np.array_equal(got, want)


def test_zero_rows():
    out = bs.scales_swizzle(torch.empty((0, 8), dtype=torch.uint8, device="cuda"))
    assert out.numel() == 0

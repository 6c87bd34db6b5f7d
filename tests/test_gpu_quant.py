"""GPU parity: fp4_quantize and fp4_global_scale against the oracle, bit-exact.

Inputs are seeded and synthetic (block_scaled_fp4_e2m1_amd.synth); the
expected bytes come from oracle/quant.py.  Shapes span several launch waves
and ragged tails, plus the degenerate blocks of the method (zeros, signed
zeros, single values, subnormal and saturating scales).
"""
import numpy as np
import pytest
import torch

import block_scaled_fp4_e2m1_amd as bs
from block_scaled_fp4_e2m1_amd import synth
from oracle import formats as F
from oracle import moe as OM
from oracle import quant as OQ

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def _host(t):
    return t.cpu().numpy()


def _gpu_nvfp4(bits, gs):
    x = _dev_bf16(bits)
    g = torch.tensor([gs], dtype=torch.float32, device=DEV)
    q, sf = bs.quantize(x, "nvfp4", gs=g)
    torch.cuda.synchronize()
    return _host(q), _host(sf)


def _gpu_mxfp4(bits, row_map=None):
    x = _dev_bf16(bits)
    rm = None if row_map is None else torch.from_numpy(np.asarray(row_map, np.int32)).to(DEV)
    q, sf = bs.quantize(x, "mxfp4", row_map=rm)
    torch.cuda.synchronize()
    return _host(q), _host(sf)


def _assert_bytes_equal(got, want, what):
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{what}: {len(bad)} bytes differ, first at {bad[:5].tolist()}"


SHAPES = [(1, 16), (3, 64), (17, 160), (257, 4096), (256, 4096), (64, 7168)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("seed", [0, 1])
def test_nvfp4_quant_random(shape, seed):
    if shape[1] % 16:
        pytest.skip()
    x = synth.bf16_normal_with_outliers(100 + seed, 200 + seed, shape)
    gs = OQ.global_scale(x)
    q, sf = _gpu_nvfp4(x, gs)
    wq, wsf = OQ.nvfp4_quantize(x, gs)
    _assert_bytes_equal(sf, wsf, f"sf {shape}")
    _assert_bytes_equal(q, wq, f"q {shape}")


@pytest.mark.parametrize("shape", [(1, 32), (5, 96), (33, 2048), (300, 4096)])
def test_mxfp4_quant_random(shape):
    x = synth.bf16_normal_with_outliers(300, 301, shape)
    q, sf = _gpu_mxfp4(x)
    wq, wsf = OQ.mxfp4_quantize(x)
    _assert_bytes_equal(sf, wsf, f"sf {shape}")
    _assert_bytes_equal(q, wq, f"q {shape}")


def _edge_rows():
    """Rows of 64 bf16 values covering the method's degenerate blocks."""
    rows = []
    z = np.zeros(64, np.float32)
    rows.append(z.copy())                                   # all zero
    r = z.copy(); r[::2] = -0.0; rows.append(r)             # signed zeros
    r = z.copy(); r[5] = 3.0; r[40] = -1e-3; rows.append(r)  # single values
    r = np.full(64, 2.0 ** -133, np.float32); r[1::2] *= -1; rows.append(r)  # bf16 subnormals
    r = np.full(64, 1e-30, np.float32); rows.append(r)      # scale underflows to 0
    r = np.full(64, 3.0e38, np.float32); r[::3] = -1.0; rows.append(r)  # huge values
    r = np.linspace(-6, 6, 64).astype(np.float32); rows.append(r)  # ramp through every code
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], np.float32)
    r = np.tile(np.concatenate([ties, -ties]), 4); rows.append(r)  # E2M1 ties at scale 1
    return synth.f32_to_bf16_bits(np.stack(rows))


@pytest.mark.parametrize("gs", [1.0, 3.0, 1.1, 4096.0, 2.0 ** -20, 2688.0])
def test_nvfp4_quant_edge_blocks(gs):
    x = _edge_rows()
    q, sf = _gpu_nvfp4(x, np.float32(gs))
    wq, wsf = OQ.nvfp4_quantize(x, np.float32(gs))
    _assert_bytes_equal(sf, wsf, "sf")
    _assert_bytes_equal(q, wq, "q")


def test_mxfp4_quant_edge_blocks():
    x = _edge_rows()
    q, sf = _gpu_mxfp4(x)
    wq, wsf = OQ.mxfp4_quantize(x)
    _assert_bytes_equal(sf, wsf, "sf")
    _assert_bytes_equal(q, wq, "q")


def test_nvfp4_scale_sweep():
    """Every E4M3 decision: block maxima swept across the whole scale range,
    with gs = 1 so that amax/6 lands on, between and around every grid point."""
    grid = F.E4M3_TABLE[:0x7F]
    mids = (grid[:-1] + grid[1:]) / 2
    s = np.concatenate([grid, mids, mids * (1 + 2 ** -10), mids * (1 - 2 ** -10)])
    amax = (s * 6).astype(np.float32)
    amax = amax[(amax > 0) & (amax < 3e38)]
    rows = np.zeros((amax.size, 16), np.float32)
    rows[:, 0] = amax
    rows[:, 1:] = amax[:, None] * np.linspace(-0.99, 0.99, 15, dtype=np.float32)[None]
    x = synth.f32_to_bf16_bits(rows)
    q, sf = _gpu_nvfp4(x, np.float32(1.0))
    wq, wsf = OQ.nvfp4_quantize(x, np.float32(1.0))
    _assert_bytes_equal(sf, wsf, "sf")
    _assert_bytes_equal(q, wq, "q")


def test_experts_quant_row_map():
    """MXFP4 experts quant of the MoE workload's activations: rows gathered by
    token in expert-sorted order."""
    T, H, E, topk = 512, 2048, 128, 8
    x = synth.bf16_normal(140, (T, H))
    ids, _ = synth.routing(141, T, E, topk)
    _, sorted_ids = OM.moe_prep(ids, E)
    tokens = sorted_ids // topk
    q, sf = _gpu_mxfp4(x, tokens)
    wq, wsf = OM.experts_quant(x, sorted_ids, topk)
    _assert_bytes_equal(sf, wsf, "sf")
    _assert_bytes_equal(q, wq, "q")


def test_row_map_out_of_range_gives_zero_rows():
    x = synth.bf16_normal(5, (4, 64))
    q, sf = _gpu_mxfp4(x, [0, -1, 7, 3])
    assert np.all(q[1] == 0) and np.all(sf[1] == 0)
    assert np.all(q[2] == 0) and np.all(sf[2] == 0)
    wq, wsf = OQ.mxfp4_quantize(x[[0, 3]])
    _assert_bytes_equal(q[[0, 3]], wq, "q")


def test_zero_rows_is_noop():
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    q, sf = bs.quantize(x, "mxfp4")
    assert q.shape == (0, 32) and sf.shape == (0, 2)


@pytest.mark.parametrize("shape", [(7,), (256, 4096), (4096, 7168), (3, 5)])
def test_global_scale(shape):
    x = synth.bf16_normal_with_outliers(400, 401, shape) if len(shape) == 2 else synth.bf16_normal(402, shape)
    gs = bs.global_scale(_dev_bf16(x))
    torch.cuda.synchronize()
    want = OQ.global_scale(x)
    assert gs.cpu().numpy().view(np.uint32)[0] == np.float32(want).view(np.uint32)

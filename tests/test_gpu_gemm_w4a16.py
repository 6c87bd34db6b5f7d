"""GPU parity: W4A16 (bf16 activations x NVFP4 weights) against the float64 oracle.

Tolerance: |D - Dref| <= 8e-3 |Dref| + 1e-3 rms(Dref) element-wise.  The
workload shapes (M = 64 and M = 1 at N = 4096, K = 7168) are checked in
full; smaller shapes cover m-tile boundaries, ragged K and M > 64 (rows
processed in chunks of 64).
"""
import numpy as np
import pytest
import torch

import block_scaled_fp4_e2m1_amd as bs
from block_scaled_fp4_e2m1_amd import synth
from oracle import gemm as OG
from oracle import quant as OQ
from oracle import tolerance as TOL
from gpu_helpers import dev_bf16, dev_f32, dev_u8, host_bf16_bits

pytestmark = pytest.mark.gpu


def _problem(M, N, K, seed):
    a = synth.bf16_normal(seed, (M, K))
    w = synth.bf16_normal(seed + 1, (N, K), 0.02)
    gw = OQ.global_scale(w)
    wq, wsf = OQ.nvfp4_quantize(w, gw)
    alpha = np.float32(np.float32(1.0) / gw)
    return a, wq, wsf, alpha


def _run_check(a, wq, wsf, alpha, rows=None):
    d = bs.w4a16_gemm(dev_bf16(a), dev_u8(wq), dev_u8(wsf), None if alpha is None else dev_f32([alpha]))
    torch.cuda.synchronize()
    got = host_bf16_bits(d)
    if rows is not None:
        got, a = got[rows], a[rows]
    want = OG.w4a16_gemm(a, wq, wsf, 1.0 if alpha is None else alpha)
    ok, worst, nbad = TOL.check_bf16(got, want)
    assert ok, f"{nbad} out of tolerance (worst {worst:.2f})"


@pytest.mark.parametrize("M,N,K", [(1, 32, 32), (3, 64, 96), (16, 128, 1056), (17, 96, 2048),
                                   (40, 64, 4128), (64, 256, 512), (100, 96, 256), (130, 64, 1024)])
def test_w4a16_shapes(M, N, K):
    _run_check(*_problem(M, N, K, 30 + M))


@pytest.mark.parametrize("M,seed", [(64, 130), (1, 131)])
def test_w4a16_workload(M, seed):
    a = synth.bf16_normal(seed, (M, 7168))
    w = synth.bf16_normal(132, (4096, 7168), 0.02)
    gw = OQ.global_scale(w)
    wq, wsf = OQ.nvfp4_quantize(w, gw)
    _run_check(a, wq, wsf, np.float32(np.float32(1.0) / gw))


@pytest.mark.parametrize("M", [8, 2])
def test_w4a16_every_scale_code_no_alpha(M):
    N, K = 64, 512
    a = synth.bf16_normal(1, (M, K), 4.0)
    wq = synth.random_bytes(2, (N, K // 2))
    wsf = synth.random_e4m3_scales(3, (N, K // 16), 0x00, 0x7F)
    _run_check(a, wq, wsf, None)


@pytest.mark.parametrize("M,N,K", [(33, 96, 1024), (64, 4096, 7168), (48, 160, 4160), (24, 160, 2048),
                                   (32, 4096, 7168)])
@pytest.mark.parametrize("mt4", ["1", "0"])
def test_w4a16_rows_17_to_64_small_m_kernels(monkeypatch, mt4, M, N, K):
    """Rows 17..64 through the chunked small-M kernels (split form with two or
    four M tiles, per-wave form), the 64-row tiled kernel switched off."""
    monkeypatch.setenv("BSFP4_W4A16_ROWS64", "0")
    monkeypatch.setenv("BSFP4_SKINNY_MT4", mt4)
    _run_check(*_problem(M, N, K, 700 + M))


@pytest.mark.parametrize("M,N,K", [(5, 128, 128), (16, 96, 1024), (33, 4096, 7168), (63, 288, 2048),
                                   (64, 160, 4224), (12, 1056, 8192), (64, 32, 128), (40, 96, 4160),
                                   (50, 4000, 5120), (36, 4096, 6144), (64, 4096, 8192),
                                   (65, 160, 2048), (100, 4096, 7168), (128, 288, 4224), (96, 96, 1024),
                                   (120, 1056, 19968)])
def test_w4a16_rows64_kernel(monkeypatch, M, N, K):
    """The row kernel forced for any 5..128 rows with K % 128 == 0:
    its 64-row and 128-row forms, partial row and column tiles, K ranges of
    one to several stages (the planner's choice); K % 128 != 0 takes the
    other small-M kernels."""
    monkeypatch.setenv("BSFP4_W4A16_ROWS64", "1")
    _run_check(*_problem(M, N, K, 720 + M))


@pytest.mark.parametrize("M,N,K,splits", [(64, 256, 8192, "1"), (40, 640, 4096, "3"), (17, 6656, 19968, ""),
                                          (33, 1024, 2048, "16"), (128, 256, 8192, "1"),
                                          (96, 640, 4096, "3"), (80, 1024, 2048, "16")])
def test_w4a16_rows64_long_ranges(monkeypatch, M, N, K, splits):
    """The row kernel, 64- and 128-row forms, with K ranges of many stages (64
    in one range, the planner's 4 x 39 at the down-projection shape) and with
    one stage per range."""
    if splits:
        monkeypatch.setenv("BSFP4_ROWS64_SPLITS", splits)
    _run_check(*_problem(M, N, K, 740 + M))


@pytest.mark.parametrize("M,N,K", [(1, 4096, 7168), (16, 288, 4160), (29, 1056, 16384)])
def test_w4a16_split_forms(M, N, K):
    """Split-K form (one or two M tiles) incl. K longer than 16 loads per lane."""
    _run_check(*_problem(M, N, K, 800 + M))


@pytest.mark.parametrize("M,N,K", [(65, 64, 64), (200, 288, 640), (256, 256, 2048), (300, 544, 1344),
                                   (513, 800, 4096), (1000, 96, 512)])
def test_w4a16_tiled_shapes(M, N, K):
    """Rows above 64 with K % 64 == 0: the 256 x 256 tiled kernel (ragged M and N,
    one or several tiles, K splits where tiles are few)."""
    _run_check(*_problem(M, N, K, 900 + M))


@pytest.mark.parametrize("M,N,K", [(96, 160, 1056), (130, 64, 1024 + 32)])
def test_w4a16_rows_above_64_k_not_multiple_of_64(M, N, K):
    """K % 64 != 0 keeps the 64-row chunked form."""
    _run_check(*_problem(M, N, K, 950 + M))


@pytest.mark.parametrize("M,N,K", [(4096, 4096, 7168), (512, 6656, 19968), (2048, 19968, 6656),
                                   (64, 6656, 19968), (32, 19968, 6656)])
def test_w4a16_large_sampled(M, N, K):
    """The workload shape at M = 4096 and the two projection shapes of the
    W4A16 follow-up page, checked on sampled rows (first/last tile rows included)."""
    a = synth.bf16_normal(960, (M, K))
    w = synth.bf16_normal(961, (N, K), 0.02)
    gw = OQ.global_scale(w)
    wq, wsf = OQ.nvfp4_quantize(w, gw)
    rows = np.unique(np.concatenate([[0, 255 % M, 256 % M, M - 1],
                                     np.random.default_rng(2).choice(M, 12, replace=False)]))
    _run_check(a, wq, wsf, np.float32(np.float32(1.0) / gw), rows=rows)


@pytest.mark.parametrize("M,N,K", [(1, 32, 32), (2, 96, 8192), (3, 4096, 7168), (4, 288, 4064),
                                   (1, 64, 8224), (4, 1056, 96), (2, 160, 1184)])
@pytest.mark.parametrize("form", ["few", "split"])
def test_w4a16_few_rows_forms(monkeypatch, form, M, N, K):
    """At most four rows: the LDS-staged form (activation rows copied whole into
    LDS; K tails inside a unit, K up to 8192 and just past it) and the split-K form."""
    if form == "split":
        monkeypatch.setenv("BSFP4_SKINNY_FEW", "0")
    _run_check(*_problem(M, N, K, 970 + M + K))

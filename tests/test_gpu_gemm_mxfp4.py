"""GPU parity: MXFP4 W4A4 fp4_gemm (scaled FP4 MFMA) against the float64 oracle.

Tolerance: |D - Dref| <= 8e-3 |Dref| + 1e-3 rms(Dref) element-wise.  Shapes
span several 256x256 tiles, ragged M/N, K not a multiple of the 128-value
stage, and the 4096 x 4096 x 7168 workload (sampled rows).
"""
import numpy as np
import pytest
import torch

import block_scaled_fp4_e2m1_amd as bs
from block_scaled_fp4_e2m1_amd import synth
from oracle import gemm as OG
from oracle import tolerance as TOL
from gpu_helpers import dev_f32, dev_u8, host_bf16_bits, mxfp4_problem

pytestmark = pytest.mark.gpu


def _run(aq, sfa, bq, sfb, alpha=None):
    d = bs.gemm(dev_u8(aq), dev_u8(sfa), dev_u8(bq), dev_u8(sfb),
                None if alpha is None else dev_f32([alpha]), fmt="mxfp4")
    torch.cuda.synchronize()
    return host_bf16_bits(d)


def _check(got, aq, sfa, bq, sfb, alpha=1.0, rows=None):
    if rows is None:
        ok, worst, nbad = TOL.check_bf16(got, OG.mxfp4_gemm(aq, sfa, bq, sfb, alpha))
    else:
        ok, worst, nbad = TOL.check_bf16(got[rows], OG.mxfp4_gemm(aq[rows], sfa[rows], bq, sfb, alpha))
    assert ok, f"{nbad} out of tolerance (worst {worst:.2f})"


@pytest.mark.parametrize("M,N,K", [(1, 32, 32), (7, 64, 96), (64, 256, 256), (100, 96, 160),
                                   (255, 288, 416), (256, 256, 7168), (300, 544, 1056),
                                   (513, 800, 2048)])
def test_mxfp4_gemm_random(M, N, K):
    aq, sfa, bq, sfb = mxfp4_problem(M, N, K, seed=200 + M)
    _check(_run(aq, sfa, bq, sfb), aq, sfa, bq, sfb)


def test_mxfp4_gemm_alpha_and_scale_range():
    M, N, K = 96, 128, 512
    aq = synth.random_bytes(1, (M, K // 2))
    bq = synth.random_bytes(2, (N, K // 2))
    sfa = synth.random_e8m0_scales(3, (M, K // 32), 100, 150)
    sfb = synth.random_e8m0_scales(4, (N, K // 32), 110, 140)
    alpha = np.float32(0.37)
    _check(_run(aq, sfa, bq, sfb, alpha), aq, sfa, bq, sfb, alpha)


def test_mxfp4_gemm_large_workload_sampled():
    aq, sfa, bq, sfb = mxfp4_problem(4096, 4096, 7168, seed=120)
    got = _run(aq, sfa, bq, sfb)
    rows = np.unique(np.concatenate([[0, 255, 256, 4095],
                                     np.random.default_rng(1).choice(4096, 44, replace=False)]))
    _check(got, aq, sfa, bq, sfb, rows=rows)


def test_mxfp4_gemm_deterministic():
    aq, sfa, bq, sfb = mxfp4_problem(300, 512, 1024, seed=3)
    assert np.array_equal(_run(aq, sfa, bq, sfb), _run(aq, sfa, bq, sfb))


@pytest.mark.parametrize("sg", ["0", "2", "4"])
@pytest.mark.parametrize("waves", ["4", "8"])
@pytest.mark.parametrize("M,N,K", [(300, 544, 2048), (256, 256, 1536), (77, 96, 4096)])
def test_mxfp4_gemm_loader_waves(monkeypatch, sg, waves, M, N, K):
    """Loader-wave splits of the 128-value DMA ring and both wave layouts of the dense kernel."""
    monkeypatch.setenv("BSFP4_MXFP4_RING", "128x4")
    monkeypatch.setenv("BSFP4_MXFP4_LOADERS", sg)
    monkeypatch.setenv("BSFP4_MXFP4_WAVES", waves)
    aq, sfa, bq, sfb = mxfp4_problem(M, N, K, seed=900 + M)
    _check(_run(aq, sfa, bq, sfb), aq, sfa, bq, sfb)


@pytest.mark.parametrize("ring", ["128x4", "256x2", "256x3"])
@pytest.mark.parametrize("M,N,K", [(64, 256, 256), (255, 288, 512), (513, 800, 2048), (300, 544, 1280)])
def test_mxfp4_gemm_ring_forms(monkeypatch, ring, M, N, K):
    """Every ring form of the dense kernel: 128-value stages in 4 slots, 256-value
    stages (whole 128-byte rows per DMA request) in 2 or 3 slots; K = 256 is a
    single stage, and K % 256 != 0 falls back to 128-value stages."""
    monkeypatch.setenv("BSFP4_MXFP4_RING", ring)
    aq, sfa, bq, sfb = mxfp4_problem(M, N, K, seed=950 + M)
    _check(_run(aq, sfa, bq, sfb), aq, sfa, bq, sfb)

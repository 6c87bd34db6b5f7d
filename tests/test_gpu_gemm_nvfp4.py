"""GPU parity: NVFP4 W4A4 fp4_gemm against the float64 oracle.

Tolerance (the acceptance rule of oracle/tolerance.py, checked element by
element): |D - Dref| <= 8e-3 |Dref| + 1e-3 rms(Dref), Dref = bf16(float64 result).
Shapes span several 256x256 tiles, ragged M/N/K tails, M = 1 and the
workload sizes; at the largest size the oracle computes sampled rows.
"""
import numpy as np
import pytest
import torch

import block_scaled_fp4_e2m1_amd as bs
from block_scaled_fp4_e2m1_amd import synth
from oracle import formats as F
from oracle import gemm as OG
from oracle import tolerance as TOL
from gpu_helpers import dev_f32, dev_u8, host_bf16_bits, nvfp4_problem

pytestmark = pytest.mark.gpu


def _run(aq, sfa, bq, sfb, alpha):
    d = bs.gemm(dev_u8(aq), dev_u8(sfa), dev_u8(bq), dev_u8(sfb),
                None if alpha is None else dev_f32([alpha]), fmt="nvfp4")
    torch.cuda.synchronize()
    return host_bf16_bits(d)


def _check(got, aq, sfa, bq, sfb, alpha, rows=None):
    a = 1.0 if alpha is None else alpha
    if rows is None:
        want = OG.nvfp4_gemm(aq, sfa, bq, sfb, a)
        ok, worst, nbad = TOL.check_bf16(got, want)
    else:
        want = OG.nvfp4_gemm(aq[rows], sfa[rows], bq, sfb, a)
        ok, worst, nbad = TOL.check_bf16(got[rows], want)
    assert ok, f"{nbad} elements out of tolerance (worst ratio {worst:.2f})"
    return worst


SHAPES = [
    # small-M split-K path (M <= 64): m-tile boundaries, ragged K slices, K % 256 != 0
    (1, 32, 32), (5, 64, 96), (16, 96, 1056), (17, 64, 2080), (32, 32, 128), (33, 160, 1024),
    (63, 128, 9216), (64, 256, 256),
    # tiled path (M > 64)
    (65, 96, 160), (255, 288, 416), (256, 256, 7168), (300, 544, 1056), (513, 768, 2048),
]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_nvfp4_gemm_random(M, N, K):
    aq, sfa, bq, sfb, alpha = nvfp4_problem(M, N, K, seed=10 + M)
    got = _run(aq, sfa, bq, sfb, alpha)
    _check(got, aq, sfa, bq, sfb, alpha)


@pytest.mark.parametrize("M", [16, 24, 96])
def test_nvfp4_gemm_every_scale_code(M):
    """Random codes with every finite E4M3 scale code (incl. subnormal scales)."""
    N, K = 160, 512
    aq = synth.random_bytes(1, (M, K // 2))
    bq = synth.random_bytes(2, (N, K // 2))
    sfa = synth.random_e4m3_scales(3, (M, K // 16), 0x00, 0x7F)
    sfb = synth.random_e4m3_scales(4, (N, K // 16), 0x00, 0x50)
    got = _run(aq, sfa, bq, sfb, np.float32(0.01))
    _check(got, aq, sfa, bq, sfb, np.float32(0.01))


@pytest.mark.parametrize("M", [64, 16])
def test_nvfp4_gemm_zero_blocks_and_no_alpha(M):
    N, K = 96, 256
    aq, sfa, bq, sfb, _ = nvfp4_problem(M, N, K, seed=5)
    aq[:, 32:64] = 0          # zero a whole 64-element K range in A
    sfb[:, 3] = 0             # zero scale block in B
    got = _run(aq, sfa, bq, sfb, None)
    _check(got, aq, sfa, bq, sfb, None)


def test_nvfp4_gemm_small_m_workload():
    """The memory-bound workload shape: M=16, N=4096, K=7168 (full check)."""
    aq, sfa, bq, sfb, alpha = nvfp4_problem(16, 4096, 7168, seed=100)
    got = _run(aq, sfa, bq, sfb, alpha)
    _check(got, aq, sfa, bq, sfb, alpha)


@pytest.mark.parametrize("M", [1, 64])
def test_nvfp4_gemm_sweep_small(M):
    aq, sfa, bq, sfb, alpha = nvfp4_problem(M, 4096, 7168, seed=122 + M)
    got = _run(aq, sfa, bq, sfb, alpha)
    _check(got, aq, sfa, bq, sfb, alpha)


@pytest.mark.parametrize("M,N,K,seed", [(512, 4096, 7168, 124), (2048, 4096, 7168, 125),
                                        (256, 14336, 4096, 110), (128, 4096, 7168, 126)])
def test_nvfp4_gemm_split_k_shapes(M, N, K, seed):
    """Mid-M shapes run with 128x128 tiles and/or a K split reduced in FP32."""
    aq, sfa, bq, sfb, alpha = nvfp4_problem(M, N, K, seed=seed, b_std=0.02)
    got = _run(aq, sfa, bq, sfb, alpha)
    rows = None if M <= 512 else np.unique(np.concatenate([[0, M - 1],
                                                           np.random.default_rng(2).choice(M, 62, replace=False)]))
    _check(got, aq, sfa, bq, sfb, alpha, rows=rows)


def test_nvfp4_gemm_split_k_deterministic():
    aq, sfa, bq, sfb, alpha = nvfp4_problem(256, 256, 7168, seed=8)
    assert np.array_equal(_run(aq, sfa, bq, sfb, alpha), _run(aq, sfa, bq, sfb, alpha))


def test_nvfp4_gemm_large_workload_sampled():
    """4096 x 4096 x 7168: every output of 48 sampled rows (incl. first/last)."""
    aq, sfa, bq, sfb, alpha = nvfp4_problem(4096, 4096, 7168, seed=120)
    got = _run(aq, sfa, bq, sfb, alpha)
    rows = np.unique(np.concatenate([[0, 255, 256, 4095],
                                     np.random.default_rng(0).choice(4096, 44, replace=False)]))
    _check(got, aq, sfa, bq, sfb, alpha, rows=rows)


def test_nvfp4_gemm_deterministic():
    aq, sfa, bq, sfb, alpha = nvfp4_problem(300, 512, 1024, seed=7)
    g1 = _run(aq, sfa, bq, sfb, alpha)
    g2 = _run(aq, sfa, bq, sfb, alpha)
    assert np.array_equal(g1, g2)


def test_nvfp4_gemm_m_zero():
    d = bs.gemm(dev_u8(np.zeros((0, 16), np.uint8)), dev_u8(np.zeros((0, 2), np.uint8)),
                dev_u8(np.zeros((32, 16), np.uint8)), dev_u8(np.zeros((32, 2), np.uint8)))
    assert d.shape == (0, 32)


@pytest.mark.parametrize("M", [37, 77])
def test_nvfp4_gemm_output_guard_band(M):
    """Writes stay inside D: canaries around a ragged output are untouched."""
    N, K = 96, 160
    aq, sfa, bq, sfb, alpha = nvfp4_problem(M, N, K, seed=9)
    buf = torch.full((M * N + 2 * 4096,), 0x7E57, dtype=torch.int16, device="cuda:0")
    out = buf[4096:4096 + M * N].view(M, N).view(torch.bfloat16)
    bs.gemm(dev_u8(aq), dev_u8(sfa), dev_u8(bq), dev_u8(sfb), dev_f32([alpha]), out=out)
    torch.cuda.synchronize()
    h = buf.cpu().numpy()
    assert np.all(h[:4096] == 0x7E57) and np.all(h[4096 + M * N:] == 0x7E57)
    _check(host_bf16_bits(out), aq, sfa, bq, sfb, alpha)


# The 256x256 kernels (dequantise-once and register-dequant forms) forced onto
# ragged shapes: partial tiles in M and N, K not a multiple of the 64/128 stage,
# odd numbers of K stages per split, and several split counts.
FORCED = [
    # (M, N, K, splits)
    (65, 96, 160, 1), (300, 544, 1056, 1), (257, 288, 96, 1), (513, 768, 2048, 3),
    (256, 256, 7168, 1), (300, 288, 1088, 2), (97, 1056, 4160, 5),
]


@pytest.mark.parametrize("variant", ["", "w8", "lds4", "reg8", "reg4"])
@pytest.mark.parametrize("M,N,K,splits", FORCED)
def test_nvfp4_gemm_forced_256_tiles(monkeypatch, variant, M, N, K, splits):
    monkeypatch.setenv("BSFP4_NVFP4_TILE", "256")
    monkeypatch.setenv("BSFP4_NVFP4_SPLITS", str(splits))
    if variant:
        monkeypatch.setenv("BSFP4_NVFP4_KERNEL", variant)
    aq, sfa, bq, sfb, alpha = nvfp4_problem(M, N, K, seed=300 + M + splits)
    got = _run(aq, sfa, bq, sfb, alpha)
    _check(got, aq, sfa, bq, sfb, alpha)


@pytest.mark.parametrize("tile", ["128", "256x128"])
@pytest.mark.parametrize("variant", ["", "w8", "reg8"])
@pytest.mark.parametrize("M,N,K,splits", [(300, 544, 1056, 1), (513, 768, 2048, 3), (97, 1056, 4160, 5),
                                          (257, 288, 96, 1), (129, 160, 3072, 2)])
def test_nvfp4_gemm_forced_other_tiles(monkeypatch, tile, variant, M, N, K, splits):
    if variant.startswith("reg") and tile == "256x128":
        pytest.skip("the register-dequant kernels have no 256x128 tile")
    monkeypatch.setenv("BSFP4_NVFP4_TILE", tile)
    if variant:
        monkeypatch.setenv("BSFP4_NVFP4_KERNEL", variant)
    monkeypatch.setenv("BSFP4_NVFP4_SPLITS", str(splits))
    aq, sfa, bq, sfb, alpha = nvfp4_problem(M, N, K, seed=400 + M)
    got = _run(aq, sfa, bq, sfb, alpha)
    _check(got, aq, sfa, bq, sfb, alpha)


@pytest.mark.parametrize("M,N,K", [(1, 64, 128), (3, 96, 4000 - 4000 % 32), (16, 4096, 7168), (9, 1056, 16384),
                                   (16, 288, 32), (5, 160, 1088), (16, 128, 8192), (2, 96, 8224),
                                   (11, 4096, 4064), (16, 64, 96), (7, 1056, 2304), (1, 32, 256),
                                   (4, 4096, 4032), (8, 288, 1056), (13, 160, 3840)])
@pytest.mark.parametrize("form", ["few", "lds", "onepass", "split"])
def test_nvfp4_gemm_small_m_forms(monkeypatch, form, M, N, K):
    """The small-M forms (few-row and 16-row LDS-staged, register single pass,
    split-K + reduce) on ragged shapes: K tails inside a 128-value unit, K up to
    the LDS forms' 8192 limit and just past it, several wave counts and units
    per wave, the 16-row form's per-wave scale copies (K % 256 == 0) and its
    whole-block copy (shapes outside a form's conditions take the next form)."""
    if form != "few":
        monkeypatch.setenv("BSFP4_SKINNY_FEW", "0")
    if form == "onepass":
        monkeypatch.setenv("BSFP4_SKINNY_LDS", "0")
    if form == "split":
        monkeypatch.setenv("BSFP4_SKINNY_SPLIT", "1")
    aq, sfa, bq, sfb, alpha = nvfp4_problem(M, N, K, seed=500 + M + K)
    got = _run(aq, sfa, bq, sfb, alpha)
    _check(got, aq, sfa, bq, sfb, alpha)


@pytest.mark.parametrize("M,N,K", [(1, 64, 128), (2, 96, 4064), (1, 4096, 7168), (2, 4096, 7168),
                                   (1, 32, 32), (2, 288, 8192), (1, 1056, 96), (2, 160, 1056)])
@pytest.mark.parametrize("form", ["1", "0"])
def test_nvfp4_gemm_few_rows_fp4_mfma(monkeypatch, form, M, N, K):
    """One or two rows on the scaled FP4 MFMA (block-diagonal activation operand,
    per-block E4M3 scales applied to the exact block dot products; the default)
    and on the dequantising form."""
    monkeypatch.setenv("BSFP4_FEW_FP4MFMA", form)
    aq, sfa, bq, sfb, alpha = nvfp4_problem(M, N, K, seed=600 + M + K)
    got = _run(aq, sfa, bq, sfb, alpha)
    _check(got, aq, sfa, bq, sfb, alpha)


@pytest.mark.parametrize("M,N,K", [(33, 96, 1024), (64, 4096, 7168), (48, 160, 4160), (24, 160, 2048),
                                   (32, 4096, 7168)])
@pytest.mark.parametrize("mt4", ["1", "0"])
def test_nvfp4_gemm_rows_17_to_64_small_m_kernels(monkeypatch, mt4, M, N, K):
    """Rows 17..64 through the chunked small-M kernels (split form with two or
    four M tiles, per-wave form), the 64-row kernel switched off."""
    monkeypatch.setenv("BSFP4_NVFP4_ROWS64", "0")
    monkeypatch.setenv("BSFP4_SKINNY_MT4", mt4)
    aq, sfa, bq, sfb, alpha = nvfp4_problem(M, N, K, seed=600 + M)
    got = _run(aq, sfa, bq, sfb, alpha)
    _check(got, aq, sfa, bq, sfb, alpha)


@pytest.mark.parametrize("M,N,K", [(5, 128, 128), (16, 96, 1024), (33, 4096, 7168), (63, 288, 2048),
                                   (64, 160, 4224), (12, 1056, 8192), (64, 32, 128), (40, 96, 4160),
                                   (50, 4000, 5120), (36, 4096, 6144), (64, 4096, 8192), (47, 4096, 7168),
                                   (65, 160, 2048), (100, 4096, 7168), (128, 288, 4224), (96, 96, 1024),
                                   (120, 1056, 19968)])
def test_nvfp4_gemm_rows64_kernel(monkeypatch, M, N, K):
    """The row kernel with NVFP4 activations forced for any 5..128 rows with K % 128 == 0:
    its 64-row and 128-row forms, partial row and column tiles, K ranges of
    one to several stages (the planner's choice); K % 128 != 0 takes the
    other small-M kernels."""
    monkeypatch.setenv("BSFP4_NVFP4_ROWS64", "1")
    aq, sfa, bq, sfb, alpha = nvfp4_problem(M, N, K, seed=640 + M)
    got = _run(aq, sfa, bq, sfb, alpha)
    _check(got, aq, sfa, bq, sfb, alpha)


@pytest.mark.parametrize("M,N,K,splits", [(64, 256, 8192, "1"), (40, 640, 4096, "3"), (17, 6656, 19968, ""),
                                          (33, 1024, 2048, "16"), (128, 256, 8192, "1"),
                                          (96, 640, 4096, "3"), (80, 1024, 2048, "16")])
def test_nvfp4_gemm_rows64_long_ranges(monkeypatch, M, N, K, splits):
    """The row kernel (NVFP4 activations), 64- and 128-row forms, with K
    ranges of many stages and with one stage per range."""
    if splits:
        monkeypatch.setenv("BSFP4_ROWS64_SPLITS", splits)
    aq, sfa, bq, sfb, alpha = nvfp4_problem(M, N, K, seed=680 + M)
    got = _run(aq, sfa, bq, sfb, alpha)
    _check(got, aq, sfa, bq, sfb, alpha)


def test_nvfp4_gemm_rows64_every_scale_code():
    """Every E4M3 scale code on both operands (incl. subnormal codes and zero)
    through the 64-row kernel's fp16 dequantisation."""
    M, N, K = 64, 256, 2048
    aq = synth.random_bytes(661, (M, K // 2))
    bq = synth.random_bytes(662, (N, K // 2))
    sfa = (np.arange(M * (K // 16)) % 0x7F).astype(np.uint8).reshape(M, K // 16)
    sfb = ((np.arange(N * (K // 16)) * 5 + 3) % 0x7F).astype(np.uint8).reshape(N, K // 16)
    got = _run(aq, sfa, bq, sfb, None)
    _check(got, aq, sfa, bq, sfb, None)

"""Pins for oracle/gemm.py: NVFP4, MXFP4 and W4A16 GEMMs.

Pins: hand-worked dot products (tests/golden/gemm_examples.json); exact
brute force with Python integers and Fractions on tiny non-square shapes
(catches a transposed operand, a wrong scale index or a dropped block);
scale-doubling and alpha-linearity identities; K-block permutation
invariance; zero blocks; and cross-path identities (W4A16 on exactly
representable activations equals W4A4; NVFP4 with power-of-two scales equal
within 32-element pairs equals MXFP4).
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from block_scaled_fp4_e2m1_amd import synth
from oracle import formats as F
from oracle import gemm as G
from oracle import quant as Q


@pytest.fixture(scope="module")
def examples(golden_dir):
    with open(os.path.join(golden_dir, "gemm_examples.json")) as f:
        return json.load(f)


def _pack(codes):
    return F.pack_nibbles(np.asarray(codes, dtype=np.uint8))


# ---------------------------------------------------------------- golden

def test_golden_nvfp4(examples):
    for ex in examples["nvfp4"]:
        a = _pack([[2] * 32])
        b = _pack([[7] * 16 + [9] * 16])
        sfa = np.array([[int(s, 16) for s in ex["sfa"]]], np.uint8)
        sfb = np.array([[int(s, 16) for s in ex["sfb"]]], np.uint8)
        d = G.nvfp4_gemm(a, sfa, b, sfb, np.float32(ex["alpha"]))
        assert f"{int(d[0, 0]):04x}" == ex["d_bf16_hex"], ex["name"]


def test_golden_mxfp4(examples):
    ex = examples["mxfp4"][0]
    d = G.mxfp4_gemm(_pack([[4] * 32]), np.array([ex["sfa"]], np.uint8),
                     _pack([[5] * 32]), np.array([ex["sfb"]], np.uint8))
    assert f"{int(d[0, 0]):04x}" == ex["d_bf16_hex"]


# ---------------------------------------------------------------- brute force

_E2M1_TWICE = [0, 1, 2, 3, 4, 6, 8, 12]          # 2 * |e2m1| as integers


def _e2m1_frac(c):
    v = Fraction(_E2M1_TWICE[c & 7], 2)
    return -v if c & 8 else v


def _e4m3_frac(c):
    e, m = (c >> 3) & 0xF, c & 7
    if e == 0:
        return Fraction(m, 8) * Fraction(1, 64)
    return (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)


def _bf16_of_fraction(x: Fraction) -> float:
    if x == 0:
        return 0.0
    a = abs(x)
    e = 0
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = Fraction(2) ** (e - 7)
    r = round(a / q) * q
    return float(r) if x > 0 else -float(r)


def _brute(a_codes, a_scale, b_codes, b_scale, blk, alpha, a_vals=None):
    M = len(a_scale) if a_vals is None else len(a_vals)
    N, K = len(b_codes), len(b_codes[0])
    out = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                av = a_vals[m][k] if a_vals is not None else \
                    _e2m1_frac(a_codes[m][k]) * a_scale[m][k // blk]
                acc += av * _e2m1_frac(b_codes[n][k]) * b_scale[n][k // blk]
            out[m, n] = _bf16_of_fraction(acc * Fraction(float(np.float32(alpha))))
    return out


@pytest.mark.parametrize("M,N,K", [(3, 5, 32), (7, 2, 64), (1, 9, 48)])
def test_nvfp4_brute_force(M, N, K):
    ac = synth.random_bytes(10 + M, (M, K)) & 0xF
    bc = synth.random_bytes(20 + N, (N, K)) & 0xF
    sfa = synth.random_e4m3_scales(30, (M, K // 16), 0x01, 0x7F)
    sfb = synth.random_e4m3_scales(31, (N, K // 16), 0x01, 0x7F)
    alpha = np.float32(0.3)
    got = F.bf16_bits_to_f64(G.nvfp4_gemm(_pack(ac), sfa, _pack(bc), sfb, alpha))
    want = _brute(ac.tolist(), [[_e4m3_frac(int(s)) for s in r] for r in sfa],
                  bc.tolist(), [[_e4m3_frac(int(s)) for s in r] for r in sfb], 16, alpha)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("M,N,K", [(4, 3, 64), (2, 6, 32)])
def test_mxfp4_brute_force(M, N, K):
    ac = synth.random_bytes(40, (M, K)) & 0xF
    bc = synth.random_bytes(41, (N, K)) & 0xF
    sfa = synth.random_e8m0_scales(42, (M, K // 32))
    sfb = synth.random_e8m0_scales(43, (N, K // 32))
    got = F.bf16_bits_to_f64(G.mxfp4_gemm(_pack(ac), sfa, _pack(bc), sfb))
    p2 = lambda c: Fraction(2) ** (int(c) - 127)
    want = _brute(ac.tolist(), [[p2(s) for s in r] for r in sfa],
                  bc.tolist(), [[p2(s) for s in r] for r in sfb], 32, 1.0)
    assert np.array_equal(got, want)


def test_w4a16_brute_force():
    M, N, K = 3, 4, 32
    a = synth.bf16_normal(50, (M, K))
    bc = synth.random_bytes(51, (N, K)) & 0xF
    sfb = synth.random_e4m3_scales(52, (N, K // 16))
    alpha = np.float32(1.7)
    got = F.bf16_bits_to_f64(G.w4a16_gemm(a, _pack(bc), sfb, alpha))
    av = [[Fraction(float(t)) for t in row] for row in F.bf16_bits_to_f32(a)]
    want = _brute(None, None, bc.tolist(), [[_e4m3_frac(int(s)) for s in r] for r in sfb],
                  16, alpha, a_vals=av)
    assert np.array_equal(got, want)


# ---------------------------------------------------------------- identities

def _rand_nvfp4(seed, M, N, K):
    a = synth.bf16_normal(seed, (M, K))
    b = synth.bf16_normal(seed + 1, (N, K), 0.02)
    ga, gb = Q.global_scale(a), Q.global_scale(b)
    aq, sfa = Q.nvfp4_quantize(a, ga)
    bq, sfb = Q.nvfp4_quantize(b, gb)
    alpha = np.float32(np.float32(1.0) / np.float32(ga * gb))
    return aq, sfa, bq, sfb, alpha


def test_scale_doubling_doubles_output():
    M, N, K = 8, 16, 128
    aq = _pack(synth.random_bytes(60, (M, K)) & 0xF)
    bq = _pack(synth.random_bytes(61, (N, K)) & 0xF)
    sfa = synth.random_e4m3_scales(62, (M, K // 16))
    sfb = synth.random_e4m3_scales(63, (N, K // 16))
    ref = G.nvfp4_gemm_f64(aq, sfa, bq, sfb, 0.75)
    got = G.nvfp4_gemm_f64(aq, sfa + 8, bq, sfb, 0.75)   # +8 = exponent field + 1
    assert np.array_equal(got, 2 * ref)
    # doubling a single block of one row changes only that row's block term
    sfa3 = sfa.copy()
    sfa3[2, 5] += 8
    got3 = G.nvfp4_gemm_f64(aq, sfa3, bq, sfb, 0.75)
    part = G.nvfp4_gemm_f64(aq[2:3, 40:48], sfa[2:3, 5:6], bq[:, 40:48], sfb[:, 5:6], 0.75)
    assert np.allclose(got3[2] - ref[2], part[0], rtol=0, atol=1e-9 * np.abs(ref).max())
    assert np.array_equal(np.delete(got3, 2, 0), np.delete(ref, 2, 0))


def test_linear_in_alpha():
    aq, sfa, bq, sfb, _ = _rand_nvfp4(61, 4, 8, 64)
    r1 = G.nvfp4_gemm_f64(aq, sfa, bq, sfb, 1.0)
    r4 = G.nvfp4_gemm_f64(aq, sfa, bq, sfb, 0.25)
    assert np.array_equal(r4, r1 * 0.25)


def test_kblock_permutation_invariance():
    aq, sfa, bq, sfb, alpha = _rand_nvfp4(62, 4, 8, 128)
    perm = np.random.default_rng(0).permutation(8)
    byte_perm = (perm[:, None] * 8 + np.arange(8)[None]).reshape(-1)
    r0 = G.nvfp4_gemm(aq, sfa, bq, sfb, alpha)
    r1 = G.nvfp4_gemm(aq[:, byte_perm], sfa[:, perm], bq[:, byte_perm], sfb[:, perm], alpha)
    assert np.array_equal(r0, r1)


def test_zero_blocks_contribute_nothing():
    aq, sfa, bq, sfb, alpha = _rand_nvfp4(63, 4, 8, 64)
    r_half = G.nvfp4_gemm_f64(aq[:, :16], sfa[:, :2], bq[:, :16], sfb[:, :2], alpha)
    aq2 = aq.copy()
    aq2[:, 16:] = 0
    assert np.array_equal(G.nvfp4_gemm_f64(aq2, sfa, bq, sfb, alpha), r_half)


def test_w4a16_equals_w4a4_on_exact_activations():
    aq, sfa, bq, sfb, _ = _rand_nvfp4(64, 8, 8, 128)
    a_vals = Q.nvfp4_dequantize(aq, sfa)                  # 6-bit products: exact in bf16
    a_bits = synth.f32_to_bf16_bits(a_vals.astype(np.float32))
    assert np.array_equal(F.bf16_bits_to_f64(a_bits), a_vals)
    assert np.array_equal(G.w4a16_gemm_f64(a_bits, bq, sfb, 0.5),
                          G.nvfp4_gemm_f64(aq, sfa, bq, sfb, 0.5))


def test_nvfp4_with_pow2_pair_scales_equals_mxfp4():
    M, N, K = 4, 6, 128
    ac = synth.random_bytes(70, (M, K)) & 0xF
    bc = synth.random_bytes(71, (N, K)) & 0xF
    ea = synth.random_e8m0_scales(72, (M, K // 32), 124, 131)
    eb = synth.random_e8m0_scales(73, (N, K // 32), 124, 131)
    # E4M3 code of 2**(c-127) is (c-127+7) << 3, duplicated for both halves
    to_e4 = lambda e: np.repeat(((e.astype(int) - 120) << 3).astype(np.uint8), 2, axis=1)
    nv = G.nvfp4_gemm_f64(_pack(ac), to_e4(ea), _pack(bc), to_e4(eb), 1.0)
    mx = G.mxfp4_gemm_f64(_pack(ac), ea, _pack(bc), eb)
    assert np.array_equal(nv, mx)

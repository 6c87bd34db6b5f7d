"""Pins for oracle/moe.py: routing prep, SiLU-gate, combine and the layer.

Pins: a brute-force per-token loop for the expert grouping; the top-1,
single-expert case, where the layer reduces to a dense MXFP4 GEMM chain
computed with the dense oracle GEMMs; SiLU against scalar math.exp
evaluations and its closed forms; the combine against exact Fractions; and
experts that receive no rows.
"""
import math
from fractions import Fraction

import numpy as np

from block_scaled_fp4_e2m1_amd import synth
from oracle import formats as F
from oracle import gemm as G
from oracle import moe as MOE
from oracle import quant as Q


def test_moe_prep_brute_force():
    ids, _ = synth.routing(1, 50, 12, 3)
    offsets, sorted_ids = MOE.moe_prep(ids, 12)
    rows = []
    for e in range(12):
        for t in range(50):
            for j in range(3):
                if ids[t, j] == e:
                    rows.append(t * 3 + j)
    assert sorted_ids.tolist() == rows
    counts = [int(np.sum(ids == e)) for e in range(12)]
    assert offsets.tolist() == [0] + list(np.cumsum(counts))


def test_routing_is_topk_of_softmax():
    ids, w = synth.routing(2, 20, 16, 4)
    assert np.all(np.diff(w, axis=1) <= 0)
    assert np.all([len(set(r)) == 4 for r in ids.tolist()])
    assert np.all(w.sum(axis=1) < 1.0)


def _weights(seed, E, N, K):
    w = synth.bf16_normal(seed, (E * N, K), 0.02)
    q, sf = Q.mxfp4_quantize(w)
    return q.reshape(E, N, K // 2), sf.reshape(E, N, K // 32)


def test_single_expert_top1_reduces_to_dense_chain():
    T, H, I, E = 24, 64, 32, 3
    x = synth.bf16_normal(3, (T, H))
    ids = np.full((T, 1), 1, np.int32)
    w = np.full((T, 1), 0.5, np.float32)
    W13q, W13sf = _weights(4, E, 2 * I, H)
    W2q, W2sf = _weights(5, E, H, I)
    st = MOE.moe_layer(x, ids, w, W13q, W13sf, W2q, W2sf)
    xq, xsf = Q.mxfp4_quantize(x)
    h1 = G.mxfp4_gemm(xq, xsf, W13q[1], W13sf[1])
    assert np.array_equal(st["h1"], h1)
    g = F.bf16_bits_to_f64(h1[:, :I])
    u = F.bf16_bits_to_f64(h1[:, I:])
    act = F.bf16_rne_from_f64(g / (1 + np.exp(-g)) * u)
    aq, asf = Q.mxfp4_quantize(act)
    y = G.mxfp4_gemm_f64(aq, asf, W2q[1], W2sf[1])
    assert np.array_equal(st["out"], F.bf16_rne_from_f64(0.5 * y))
    assert st["offsets"].tolist() == [0, 0, T, T]


def test_silu_mul_scalar():
    h = synth.bf16_normal(6, (5, 16), 3.0)
    act = F.bf16_bits_to_f64(MOE.silu_mul(h))
    hv = F.bf16_bits_to_f64(h)
    for r in range(5):
        for c in range(8):
            g, u = float(hv[r, c]), float(hv[r, c + 8])
            want = F.bf16_bits_to_f64(F.bf16_rne_from_f64(g / (1.0 + math.exp(-g)) * u))
            assert act[r, c] == want
    z = np.zeros((1, 4), np.uint16)            # silu(0) * u = 0
    assert np.all(F.bf16_bits_to_f64(MOE.silu_mul(z)) == 0)


def test_combine_exact():
    T, topk, N = 6, 2, 5
    ids, w = synth.routing(7, T, 4, topk)
    _, sorted_ids = MOE.moe_prep(ids, 4)
    Y = np.random.default_rng(8).standard_normal((T * topk, N))
    out = F.bf16_bits_to_f64(MOE.combine(Y, sorted_ids, w, T))
    for t in range(T):
        for n in range(N):
            acc = Fraction(0)
            for r, f in enumerate(sorted_ids.tolist()):
                if f // topk == t:
                    acc += Fraction(float(w[t, f % topk])) * Fraction(float(Y[r, n]))
            want = float(F.bf16_bits_to_f64(F.bf16_rne_from_f64(float(acc))))
            assert abs(out[t, n] - want) == 0 or abs(float(acc) - out[t, n]) <= abs(want) * 2 ** -8


def test_empty_experts():
    T, H, I, E = 16, 32, 32, 6
    x = synth.bf16_normal(9, (T, H))
    ids = np.stack([np.full(T, 0), np.full(T, 4)], axis=1).astype(np.int32)
    w = np.full((T, 2), 0.25, np.float32)
    W13q, W13sf = _weights(10, E, 2 * I, H)
    W2q, W2sf = _weights(11, E, H, I)
    st = MOE.moe_layer(x, ids, w, W13q, W13sf, W2q, W2sf)
    assert st["offsets"].tolist() == [0, T, T, T, T, 2 * T, 2 * T]
    # scrambling the unused experts' weights changes nothing
    W13q2 = W13q.copy()
    W13q2[[1, 2, 3, 5]] ^= 0x5A
    st2 = MOE.moe_layer(x, ids, w, W13q2, W13sf, W2q, W2sf)
    assert np.array_equal(st["out"], st2["out"])

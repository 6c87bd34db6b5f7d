"""Pins for the NVFP4 form of the mixture-of-experts layer in oracle/moe.py.

Pins: a per-token, per-slot loop that never sorts rows (each routed pair
quantised, multiplied and re-quantised on its own with the dense NVFP4
oracle, which has its own pins), checked stage by stage; the top-1,
single-expert case, where the layer is the dense NVFP4 chain; the scale
covariance of the NVFP4 encoding (doubling one expert's global scale and
halving its alpha leaves every output unchanged while no block scale leaves
the normal E4M3 range), which fails if a global scale or alpha is taken from
the wrong expert; and experts that receive no rows.
"""
import numpy as np

from block_scaled_fp4_e2m1_amd import synth
from oracle import formats as F
from oracle import gemm as G
from oracle import moe as MOE
from oracle import quant as Q


def _experts(seed, E, N, K):
    """Per-expert NVFP4 weights, each with its own global scale."""
    w = synth.bf16_normal(seed, (E, N, K), 0.02)
    q = np.zeros((E, N, K // 2), np.uint8)
    sf = np.zeros((E, N, K // 16), np.uint8)
    gsw = np.zeros(E, np.float32)
    for e in range(E):
        gsw[e] = Q.global_scale(w[e])
        q[e], sf[e] = Q.nvfp4_quantize(w[e], gsw[e])
    return q, sf, gsw


def _layer_inputs(T=20, H=64, I=32, E=5, topk=2, seed=0):
    x = synth.bf16_normal(seed + 1, (T, H))
    ids, w = synth.routing(seed + 2, T, E, topk)
    W13q, W13sf, gw13 = _experts(seed + 3, E, 2 * I, H)
    W2q, W2sf, gw2 = _experts(seed + 4, E, H, I)
    gx = Q.global_scale(x)
    # distinct per-expert activation scales and alphas
    gs1 = (gx * np.float32(2.0) ** -np.arange(E) * np.float32(0.9)).astype(np.float32)
    gs2 = (np.float32(40.0) * (1 + np.arange(E, dtype=np.float32) / 7)).astype(np.float32)
    alpha1 = (np.float32(1.0) / (gs1 * gw13)).astype(np.float32)
    alpha2 = (np.float32(1.0) / (gs2 * gw2)).astype(np.float32)
    return x, ids, w, W13q, W13sf, W2q, W2sf, gs1, alpha1, gs2, alpha2


def test_per_pair_loop_matches_layer():
    args = _layer_inputs()
    x, ids, w, W13q, W13sf, W2q, W2sf, gs1, alpha1, gs2, alpha2 = args
    st = MOE.nvfp4_moe_layer(*args)
    T, topk = ids.shape
    I = W2q.shape[2] * 2
    row_of = {int(f): r for r, f in enumerate(st["sorted_ids"])}
    out = np.zeros((T, W2q.shape[1]))
    for t in range(T):
        for j in range(topk):
            e = int(ids[t, j])
            r = row_of[t * topk + j]
            xq, xsf = Q.nvfp4_quantize(x[t:t + 1], gs1[e])
            assert np.array_equal(st["xq"][r], xq[0]) and np.array_equal(st["xsf"][r], xsf[0])
            h = G.nvfp4_gemm(xq, xsf, W13q[e], W13sf[e], alpha1[e])
            assert np.array_equal(st["h1"][r], h[0])
            hv = F.bf16_bits_to_f64(h)
            act = F.bf16_rne_from_f64(hv[:, :I] / (1 + np.exp(-hv[:, :I])) * hv[:, I:])
            assert np.array_equal(st["act"][r], act[0])
            aq, asf = Q.nvfp4_quantize(act, gs2[e])
            assert np.array_equal(st["aq"][r], aq[0]) and np.array_equal(st["asf"][r], asf[0])
            y = G.nvfp4_gemm_f64(aq, asf, W2q[e], W2sf[e], alpha2[e])
            assert np.array_equal(st["y"][r], y[0])
            out[t] += np.float64(w[t, j]) * y[0]
    got = F.bf16_bits_to_f64(st["out"])
    want = F.bf16_bits_to_f64(F.bf16_rne_from_f64(out))
    # the two float64 sums may differ in their last bit, which can move a bf16 tie
    assert np.all(np.abs(got - want) <= np.abs(want) * 2.0 ** -8)
    assert np.mean(got == want) > 0.99


def test_single_expert_top1_is_dense_chain():
    x, _, _, W13q, W13sf, W2q, W2sf, gs1, alpha1, gs2, alpha2 = _layer_inputs(T=24, E=3)
    T = x.shape[0]
    I = W2q.shape[2] * 2
    ids = np.full((T, 1), 1, np.int32)
    w = np.full((T, 1), 0.5, np.float32)
    st = MOE.nvfp4_moe_layer(x, ids, w, W13q, W13sf, W2q, W2sf, gs1, alpha1, gs2, alpha2)
    xq, xsf = Q.nvfp4_quantize(x, gs1[1])
    h1 = G.nvfp4_gemm(xq, xsf, W13q[1], W13sf[1], alpha1[1])
    assert np.array_equal(st["h1"], h1)
    g = F.bf16_bits_to_f64(h1[:, :I])
    u = F.bf16_bits_to_f64(h1[:, I:])
    aq, asf = Q.nvfp4_quantize(F.bf16_rne_from_f64(g / (1 + np.exp(-g)) * u), gs2[1])
    assert np.array_equal(st["aq"], aq) and np.array_equal(st["asf"], asf)
    y = G.nvfp4_gemm_f64(aq, asf, W2q[1], W2sf[1], alpha2[1])
    assert np.array_equal(st["out"], F.bf16_rne_from_f64(0.5 * y))
    assert st["offsets"].tolist() == [0, 0, T, T]


def _normal_range(sf):
    dec = F.E4M3_TABLE[sf]
    return bool(np.all((dec >= 2.0 ** -6) & (dec <= 224.0)))


def test_scale_covariance_per_expert():
    args = list(_layer_inputs(E=4, seed=10))
    args[7] = (args[7] * np.float32(0.5)).astype(np.float32)  # gs1: block scales <= 224
    st = MOE.nvfp4_moe_layer(*args)
    assert _normal_range(st["xsf"]) and _normal_range(st["asf"])
    for which, (gs_i, al_i) in (("gs1", (7, 8)), ("gs2", (9, 10))):
        for e in range(4):
            a2 = [np.array(v, copy=True) if i in (gs_i, al_i) else v for i, v in enumerate(args)]
            a2[gs_i][e] *= np.float32(2.0)
            a2[al_i][e] *= np.float32(0.5)
            st2 = MOE.nvfp4_moe_layer(*a2)
            rows = slice(int(st["offsets"][e]), int(st["offsets"][e + 1]))
            codes, scales = ("xq", "xsf") if which == "gs1" else ("aq", "asf")
            # codes unchanged, the expert's scale codes move up one binade
            assert np.array_equal(st2[codes], st[codes])
            assert np.array_equal(F.E4M3_TABLE[st2[scales][rows]], 2 * F.E4M3_TABLE[st[scales][rows]])
            assert np.array_equal(st2["out"], st["out"])
            # the alpha change alone (gs kept) does change the expert's rows
            a3 = [np.array(v, copy=True) if i == al_i else v for i, v in enumerate(args)]
            a3[al_i][e] *= np.float32(0.5)
            if rows.stop > rows.start:
                assert not np.array_equal(MOE.nvfp4_moe_layer(*a3)["out"], st["out"])


def test_empty_experts_and_unused_parameters():
    x, _, _, W13q, W13sf, W2q, W2sf, gs1, alpha1, gs2, alpha2 = _layer_inputs(T=16, E=6)
    T = x.shape[0]
    ids = np.stack([np.full(T, 0), np.full(T, 4)], axis=1).astype(np.int32)
    w = np.full((T, 2), 0.25, np.float32)
    st = MOE.nvfp4_moe_layer(x, ids, w, W13q, W13sf, W2q, W2sf, gs1, alpha1, gs2, alpha2)
    assert st["offsets"].tolist() == [0, T, T, T, T, 2 * T, 2 * T]
    unused = [1, 2, 3, 5]
    W13q2 = W13q.copy()
    W13q2[unused] ^= 0x5A
    g1, a1, g2, a2 = (np.array(v, copy=True) for v in (gs1, alpha1, gs2, alpha2))
    for v in (g1, a1, g2, a2):
        v[unused] = np.float32(123.0)
    st2 = MOE.nvfp4_moe_layer(x, ids, w, W13q2, W13sf, W2q, W2sf, g1, a1, g2, a2)
    assert np.array_equal(st["out"], st2["out"])

"""GPU parity: the NVFP4 W4A4 MoE layer (per-expert global scales and alphas),
stage by stage, through the C ABI.

As for the MXFP4 layer, each GPU stage is compared with the oracle applied to
the GPU's own previous stage output:
  experts quant (per-expert gs)   bit-exact
  grouped GEMM, bf16 rows         tolerance 8e-3 |ref| + 1e-3 rms(ref)
  fused SiLU-mul + NVFP4 quant    >= 99.9% identical codes and scales against
                                  the oracle on the GPU's bf16 gate_up rows;
                                  every dequantised value within one E2M1 step
  down GEMM + combine             tolerance, given the GPU's quantised act
Inputs: bf16 N(0,1) tokens, bf16 N(0, 0.02) weights quantised per expert with
that expert's own global scale; the activation scales are calibrated per
expert (2688 / amax of the rows the expert receives).
"""
import numpy as np
import pytest
import torch

import block_scaled_fp4_e2m1_amd as bs
from block_scaled_fp4_e2m1_amd import synth
from oracle import formats as F
from oracle import moe as OM
from oracle import quant as OQ
from oracle import tolerance as TOL
from gpu_helpers import dev_bf16, dev_f32, dev_i32, dev_u8, host_bf16_bits

pytestmark = pytest.mark.gpu


def _experts(seed, E, N, K):
    w = synth.bf16_normal(seed, (E, N, K), 0.02)
    q = np.zeros((E, N, K // 2), np.uint8)
    sf = np.zeros((E, N, K // 16), np.uint8)
    gsw = np.zeros(E, np.float32)
    for e in range(E):
        gsw[e] = OQ.global_scale(w[e])
        q[e], sf[e] = OQ.nvfp4_quantize(w[e], gsw[e])
    return q, sf, gsw


def _per_expert_gs(rows_bits, offsets):
    """2688 / amax over each expert's rows (1.0 for experts without rows)."""
    E = offsets.size - 1
    gs = np.ones(E, np.float32)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            gs[e] = OQ.global_scale(rows_bits[lo:hi])
    return gs


def _inputs(T, H, I, E, topk, seed):
    x = synth.bf16_normal(seed, (T, H))
    ids, w = synth.routing(seed + 1, T, E, topk)
    W13q, W13sf, g13 = _experts(seed + 2, E, 2 * I, H)
    W2q, W2sf, g2 = _experts(seed + 3, E, H, I)
    offs, sids = OM.moe_prep(ids, E)
    gs1 = _per_expert_gs(x[sids // topk], offs)
    alpha1 = (np.float32(1.0) / (gs1 * g13)).astype(np.float32)
    return dict(x=x, ids=ids, w=w, W13q=W13q, W13sf=W13sf, W2q=W2q, W2sf=W2sf, g2=g2, gs1=gs1,
                alpha1=alpha1, offs=offs, sids=sids)


CASES = [
    (64, 256, 128, 8, 2, 10),
    (200, 256, 192, 6, 3, 30),    # act width 192: three 64-column act tiles
    (150, 96, 96, 5, 2, 40),      # K = 96 (half a load group), act width 96 (1.5 act tiles)
    (300, 512, 256, 16, 4, 50),
    (48, 64, 64, 1024, 4, 80),    # the largest expert count: mostly empty experts
]


def _run(d):
    T, topk = d["ids"].shape
    E = d["W13q"].shape[0]
    offs, sids, stok = bs.moe_prep(dev_i32(d["ids"]), E)
    dW13, dW13sf = dev_u8(d["W13q"]), dev_u8(d["W13sf"])
    xq, xsf = bs.nvfp4_experts_quantize(dev_bf16(d["x"]), offs, dev_f32(d["gs1"]), row_map=stok)
    h1 = bs.nvfp4_moe_grouped_gemm(xq, xsf, offs, dW13, dW13sf, dev_f32(d["alpha1"]), bs.MOE_STORE_BF16)
    torch.cuda.synchronize()
    g = dict(offsets=offs.cpu().numpy(), xq=xq.cpu().numpy(), xsf=xsf.cpu().numpy(), h1=host_bf16_bits(h1))
    # act scales calibrated on the GPU's own gate_up rows
    gs2 = _per_expert_gs(OM.silu_mul(g["h1"]), d["offs"])
    alpha2 = (np.float32(1.0) / (gs2 * d["g2"])).astype(np.float32)
    aq, asf = bs.nvfp4_moe_grouped_gemm(xq, xsf, offs, dW13, dW13sf, dev_f32(d["alpha1"]),
                                        bs.MOE_SILU_MUL_QUANT, out_gs=dev_f32(gs2))
    out = bs.nvfp4_moe_grouped_gemm(aq, asf, offs, dev_u8(d["W2q"]), dev_u8(d["W2sf"]), dev_f32(alpha2),
                                    bs.MOE_WEIGHTED_COMBINE, sorted_ids=sids,
                                    topk_weights=dev_f32(d["w"].reshape(-1)), num_tokens=T, topk=topk)
    torch.cuda.synchronize()
    g.update(aq=aq.cpu().numpy(), asf=asf.cpu().numpy(), out=host_bf16_bits(out), gs2=gs2, alpha2=alpha2)
    return g


def _check(d, g):
    T, topk = d["ids"].shape
    offs, sids = d["offs"], d["sids"]
    assert np.array_equal(g["offsets"], offs)
    xq, xsf = OM.nvfp4_experts_quant(d["x"], sids, topk, offs, d["gs1"])
    assert np.array_equal(g["xq"], xq) and np.array_equal(g["xsf"], xsf)
    ref_h1 = F.bf16_rne_from_f64(OM.nvfp4_grouped_gemm_f64(xq, xsf, offs, d["W13q"], d["W13sf"], d["alpha1"]))
    ok, worst, nbad = TOL.check_bf16(g["h1"], ref_h1)
    assert ok, f"gate_up: {nbad} out of tolerance (worst {worst:.2f})"
    aq, asf = OM.nvfp4_rows_quant(OM.silu_mul(g["h1"]), offs, g["gs2"])
    same = np.mean(F.unpack_nibbles(g["aq"]) == F.unpack_nibbles(aq))
    assert same >= 0.999, f"only {same:.5f} of activation codes identical"
    assert np.mean(g["asf"] == asf) >= 0.999
    # dequantised act (times gs2 of the row's expert: the E4M3 grid) within one E2M1 step
    dq_g, dq_w = OQ.nvfp4_dequantize(g["aq"], g["asf"]), OQ.nvfp4_dequantize(aq, asf)
    step = np.repeat(np.maximum(F.E4M3_TABLE[g["asf"]], F.E4M3_TABLE[asf]), 16, axis=1) * 2.0
    assert np.all(np.abs(dq_g - dq_w) <= step)
    y = OM.nvfp4_grouped_gemm_f64(g["aq"], g["asf"], offs, d["W2q"], d["W2sf"], g["alpha2"])
    ref_out = OM.combine(y, sids, d["w"], T)
    ok, worst, nbad = TOL.check_bf16(g["out"], ref_out)
    assert ok, f"down+combine: {nbad} out of tolerance (worst {worst:.2f})"


@pytest.mark.parametrize("case", CASES)
def test_nvfp4_moe_stagewise(case):
    d = _inputs(*case)
    _check(d, _run(d))


def test_nvfp4_moe_empty_and_single_row_experts():
    T, H, I, E, topk = 40, 128, 64, 7, 2
    d = _inputs(T, H, I, E, topk, 60)
    ids = np.stack([np.full(T, 1), np.full(T, 4)], axis=1).astype(np.int32)
    ids[3, 0] = 6      # expert 6 receives exactly one row
    d["ids"] = ids
    d["offs"], d["sids"] = OM.moe_prep(ids, E)
    d["gs1"] = _per_expert_gs(d["x"][d["sids"] // topk], d["offs"])
    d["alpha1"] = (np.float32(1.0) / (d["gs1"] * np.float32(100.0))).astype(np.float32)
    _check(d, _run(d))


def test_nvfp4_moe_layer_binding_matches_stages():
    d = _inputs(64, 256, 128, 8, 2, 70)
    g = _run(d)
    out = bs.nvfp4_moe_layer(dev_bf16(d["x"]), dev_i32(d["ids"]), dev_f32(d["w"]), dev_u8(d["W13q"]),
                             dev_u8(d["W13sf"]), dev_u8(d["W2q"]), dev_u8(d["W2sf"]), dev_f32(d["gs1"]),
                             dev_f32(d["alpha1"]), dev_f32(g["gs2"]), dev_f32(g["alpha2"]))
    torch.cuda.synchronize()
    assert np.array_equal(host_bf16_bits(out), g["out"])


def test_nvfp4_moe_workload_stagewise():
    """4096 tokens, hidden 2048, 128 experts, top-8, intermediate 768."""
    d = _inputs(4096, 2048, 768, 128, 8, 240)
    g = _run(d)
    _check(d, g)
    full = OM.nvfp4_moe_layer(d["x"], d["ids"], d["w"], d["W13q"], d["W13sf"], d["W2q"], d["W2sf"],
                              d["gs1"], d["alpha1"], g["gs2"], g["alpha2"])["out"]
    err = F.bf16_bits_to_f64(g["out"]) - F.bf16_bits_to_f64(full)
    rel = TOL.rms(err) / TOL.rms(F.bf16_bits_to_f64(full))
    print(f"end-to-end from scratch: rms rel err {rel:.2e}")
    assert rel <= 0.02


def test_nvfp4_moe_single_expert():
    """E = 1, top-1: every row belongs to the one expert."""
    d = _inputs(40, 128, 64, 1, 1, 90)
    _check(d, _run(d))


@pytest.mark.parametrize("K", [64, 1024, 1040, 2064])
def test_nvfp4_experts_quantize_edges(K):
    """Rows whose row_map entry is out of range, and rows outside the expert
    offsets, are written as zeros; the other rows match the oracle.  K of at
    least 1024 (64 blocks) takes the one-wave-per-row form, with a partial
    last pass over the row's blocks for K = 1040 and 2064."""
    T, E = 12, 3
    x = synth.bf16_normal(91 + K, (T, K))
    offs = np.array([2, 5, 5, 9], np.int32)            # rows 0-1 and 9-10 belong to no expert
    row_map = np.array([0, 1, 2, 3, 4, 5, 6, 7, 8, 9, -1, 30], np.int32)
    gs = np.array([50.0, 20.0, 400.0], np.float32)
    q, sf = bs.nvfp4_experts_quantize(dev_bf16(x), dev_i32(offs), dev_f32(gs), row_map=dev_i32(row_map))
    torch.cuda.synchronize()
    q, sf = q.cpu().numpy(), sf.cpu().numpy()
    for r in range(len(row_map)):
        e = int(np.searchsorted(offs, r, side="right")) - 1
        src = row_map[r]
        if not (0 <= e < E and offs[e] <= r < offs[e + 1]) or not (0 <= src < T):
            assert not q[r].any() and not sf[r].any(), r
        else:
            wq, wsf = OQ.nvfp4_quantize(x[src:src + 1], gs[e])
            assert np.array_equal(q[r], wq[0]) and np.array_equal(sf[r], wsf[0]), r

"""GPU parity: the MXFP4 W4A4 MoE layer, stage by stage.

Each GPU stage is compared with the oracle applied to the GPU's own previous
stage output (a one-ulp bf16 difference upstream may flip an E2M1 code
downstream, so chaining the oracle from scratch would fail correct kernels):
  routing prep          bit-exact (offsets and stable row order)
  experts quant         bit-exact
  grouped GEMM (bf16)   tolerance 8e-3 |ref| + 1e-3 rms(ref)
  fused SiLU-mul-quant  >= 99.9% identical codes and scales against the oracle
                        applied to the GPU's bf16 gate_up output; every
                        dequantised value within one E2M1 step
  down GEMM + combine   tolerance, given the GPU's quantised activations
The from-scratch end-to-end error is reported and bounded loosely.
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
from gpu_helpers import DEV, dev_bf16, dev_f32, dev_i32, dev_u8, host_bf16_bits

pytestmark = pytest.mark.gpu


def _weights(seed, E, N, K):
    w = synth.bf16_normal(seed, (E * N, K), 0.02)
    q, sf = OQ.mxfp4_quantize(w)
    return q.reshape(E, N, K // 2), sf.reshape(E, N, K // 32)


def _layer_inputs(T, H, I, E, topk, seed):
    x = synth.bf16_normal(seed, (T, H))
    ids, w = synth.routing(seed + 1, T, E, topk)
    W13q, W13sf = _weights(seed + 2, E, 2 * I, H)
    W2q, W2sf = _weights(seed + 3, E, H, I)
    return x, ids, w, W13q, W13sf, W2q, W2sf


CASES = [
    (64, 256, 128, 8, 2, 10),
    (256, 512, 256, 16, 4, 20),
    (200, 256, 192, 6, 3, 30),   # I = 192: act width not a multiple of the 128-column tile
]


def test_moe_prep_bit_exact():
    for T, E, topk, seed in [(1, 4, 1, 1), (37, 8, 3, 2), (4096, 128, 8, 141), (1000, 300, 6, 4)]:
        ids, _ = synth.routing(seed, T, E, topk)
        offs, sids, stok = bs.moe_prep(dev_i32(ids), E)
        torch.cuda.synchronize()
        woffs, wsids = OM.moe_prep(ids, E)
        assert np.array_equal(offs.cpu().numpy(), woffs), (T, E)
        assert np.array_equal(sids.cpu().numpy(), wsids), (T, E)
        assert np.array_equal(stok.cpu().numpy(), wsids // topk), (T, E)


def test_moe_prep_skewed_and_empty_experts():
    ids = np.zeros((50, 2), np.int32)
    ids[:, 1] = 5
    ids[7, 0] = 2
    offs, sids, _ = bs.moe_prep(dev_i32(ids), 9)
    woffs, wsids = OM.moe_prep(ids, 9)
    assert np.array_equal(offs.cpu().numpy(), woffs)
    assert np.array_equal(sids.cpu().numpy(), wsids)


def _gpu_stages(x, ids, w, W13q, W13sf, W2q, W2sf):
    E = W13q.shape[0]
    T, topk = ids.shape
    offs, sids, stok = bs.moe_prep(dev_i32(ids), E)
    dx = dev_bf16(x)
    # experts quant as a row gather (one quantised row per routed pair) ...
    xq_rows, xsf_rows = bs.quantize(dx, "mxfp4", row_map=stok)
    # ... and the layer's form: each token quantised once, rows read by token
    xq_tok, xsf_tok = bs.quantize(dx, "mxfp4")
    dW13, dW13sf = dev_u8(W13q), dev_u8(W13sf)
    h1 = bs.mxfp4_moe_grouped_gemm(xq_tok, xsf_tok, offs, dW13, dW13sf, bs.MOE_STORE_BF16,
                                   a_row_index=stok)
    h1_rows = bs.mxfp4_moe_grouped_gemm(xq_rows, xsf_rows, offs, dW13, dW13sf, bs.MOE_STORE_BF16)
    aq, asf = bs.mxfp4_moe_grouped_gemm(xq_tok, xsf_tok, offs, dW13, dW13sf, bs.MOE_SILU_MUL_QUANT,
                                        a_row_index=stok)
    out = bs.mxfp4_moe_grouped_gemm(aq, asf, offs, dev_u8(W2q), dev_u8(W2sf), bs.MOE_WEIGHTED_COMBINE,
                                    sorted_ids=sids, topk_weights=dev_f32(w.reshape(-1)),
                                    num_tokens=T, topk=topk)
    torch.cuda.synchronize()
    return dict(offsets=offs.cpu().numpy(), sorted_ids=sids.cpu().numpy(), xq=xq_rows.cpu().numpy(),
                xsf=xsf_rows.cpu().numpy(), xq_tok=xq_tok.cpu().numpy(), xsf_tok=xsf_tok.cpu().numpy(),
                h1=host_bf16_bits(h1), h1_rows=host_bf16_bits(h1_rows), aq=aq.cpu().numpy(),
                asf=asf.cpu().numpy(), out=host_bf16_bits(out))


def _check_stages(x, ids, w, W13q, W13sf, W2q, W2sf, g):
    T, topk = ids.shape
    offs, sids = OM.moe_prep(ids, W13q.shape[0])
    assert np.array_equal(g["offsets"], offs) and np.array_equal(g["sorted_ids"], sids)
    xq, xsf = OM.experts_quant(x, sids, topk)
    assert np.array_equal(g["xq"], xq) and np.array_equal(g["xsf"], xsf)
    tq, tsf = OQ.mxfp4_quantize(x)
    assert np.array_equal(g["xq_tok"], tq) and np.array_equal(g["xsf_tok"], tsf)
    # reading activations by token index gives the same products as the gathered copy
    assert np.array_equal(g["h1"], g["h1_rows"])
    # gate_up GEMM on the GPU's (identical) quantised activations
    ref_h1 = F.bf16_rne_from_f64(OM.grouped_gemm_f64(g["xq"], g["xsf"], offs, W13q, W13sf))
    ok, worst, nbad = TOL.check_bf16(g["h1"], ref_h1)
    assert ok, f"gate_up: {nbad} out of tolerance (worst {worst:.2f})"
    # fused SiLU-mul + MXFP4 quant against the oracle on the GPU's own h1
    act = OM.silu_mul(g["h1"])
    aq, asf = OQ.mxfp4_quantize(act)
    codes_g, codes_w = F.unpack_nibbles(g["aq"]), F.unpack_nibbles(aq)
    same = np.mean(codes_g == codes_w)
    assert same >= 0.999, f"only {same:.5f} of activation codes identical"
    assert np.mean(g["asf"] == asf) >= 0.999
    dq_g = OQ.mxfp4_dequantize(g["aq"], g["asf"])
    dq_w = OQ.mxfp4_dequantize(aq, asf)
    step = np.repeat(F.E8M0_TABLE[np.maximum(g["asf"], asf)], 32, axis=1) * 2.0  # largest E2M1 step
    assert np.all(np.abs(dq_g - dq_w) <= step)
    # down GEMM + combine on the GPU's own quantised activations
    y = OM.grouped_gemm_f64(g["aq"], g["asf"], offs, W2q, W2sf)
    ref_out = OM.combine(y, sids, w, T)
    ok, worst, nbad = TOL.check_bf16(g["out"], ref_out)
    assert ok, f"down+combine: {nbad} out of tolerance (worst {worst:.2f})"
    return ref_out


@pytest.mark.parametrize("case", CASES)
def test_moe_stagewise(case):
    T, H, I, E, topk, seed = case
    inputs = _layer_inputs(T, H, I, E, topk, seed)
    g = _gpu_stages(*inputs)
    _check_stages(*inputs, g)


@pytest.mark.parametrize("ring", ["128x4", "256x2", "256x3"])
def test_moe_stagewise_ring_forms(monkeypatch, ring):
    """The grouped GEMMs in every ring form, on a shape where each workgroup runs
    the next; ~640 items per GEMM for 512 workgroups): 1024 tokens, hidden
    1024, intermediate 512, 32 experts, top-8."""
    monkeypatch.setenv("BSFP4_MXFP4_RING", ring)
    inputs = _layer_inputs(1024, 1024, 512, 32, 8, 77)
    g = _gpu_stages(*inputs)
    _check_stages(*inputs, g)


def test_moe_layer_binding_matches_stages():
    T, H, I, E, topk, seed = CASES[0]
    x, ids, w, W13q, W13sf, W2q, W2sf = _layer_inputs(T, H, I, E, topk, seed)
    out = bs.moe_layer(dev_bf16(x), dev_i32(ids), dev_f32(w), dev_u8(W13q), dev_u8(W13sf),
                       dev_u8(W2q), dev_u8(W2sf))
    torch.cuda.synchronize()
    full = OM.moe_layer(x, ids, w, W13q, W13sf, W2q, W2sf)["out"]
    err = F.bf16_bits_to_f64(host_bf16_bits(out)) - F.bf16_bits_to_f64(full)
    assert TOL.rms(err) <= 0.02 * TOL.rms(F.bf16_bits_to_f64(full))


def test_moe_workload_stagewise():
    """The MoE workload: 4096 tokens, hidden 2048, 128 experts, top-8, intermediate 768."""
    inputs = _layer_inputs(4096, 2048, 768, 128, 8, 140)
    g = _gpu_stages(*inputs)
    ref_out = _check_stages(*inputs, g)
    full = OM.moe_layer(*inputs)["out"]
    err = F.bf16_bits_to_f64(g["out"]) - F.bf16_bits_to_f64(full)
    rel = TOL.rms(err) / TOL.rms(F.bf16_bits_to_f64(full))
    print(f"end-to-end from scratch: rms rel err {rel:.2e}; max abs err {np.max(np.abs(err)):.3e}")
    assert rel <= 0.02
    assert ref_out.shape == (4096, 2048)

"""GPU: the entry points captured in a HIP graph.

Each composite step (the NVFP4 and MXFP4 MoE layers: routing prep, experts
quantisation, the grouped GEMMs with their epilogues and the top-k sum; the
fused quantise + GEMM; a split-K GEMM with its reduce kernel) is captured once
into a graph, then the graph is replayed several times with the program's own
eager work and synchronisations between the replays, after the captured
inputs have been overwritten with new values, and every replay is compared
bit for bit with the eager result on the same inputs.  The library issues no
memset or allocation of its own, so its kernels are safe to capture.
"""
import numpy as np
import pytest
import torch

import block_scaled_fp4_e2m1_amd as bs
from block_scaled_fp4_e2m1_amd import synth
from oracle import quant as OQ
from gpu_helpers import dev_bf16, dev_f32, dev_i32, dev_u8

pytestmark = pytest.mark.gpu


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                      # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = fn()
    return g, out


def _replays_match(g, graph_out, set_inputs, eager):
    for rep in range(3):
        set_inputs(rep)                                  # eager work between replays
        want = [t.clone() for t in eager()]
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(graph_out, want):
            assert torch.equal(a, b), f"replay {rep}"


def _nvfp4_experts(seed, E, N, K):
    w = synth.bf16_normal(seed, (E, N, K), 0.02)
    q = np.zeros((E, N, K // 2), np.uint8)
    sf = np.zeros((E, N, K // 16), np.uint8)
    for e in range(E):
        q[e], sf[e] = OQ.nvfp4_quantize(w[e], OQ.global_scale(w[e]))
    return dev_u8(q), dev_u8(sf)


@pytest.mark.parametrize("H", [256, 1024])
def test_moe_layers_in_a_graph(H):
    """Both MoE layers captured in one graph; H = 1024 gives the NVFP4 experts
    quantiser rows of 64 blocks (its one-wave-per-row form)."""
    T, I, E, topk = 96, 128, 8, 2
    x = dev_bf16(synth.bf16_normal(1, (T, H)))
    ids_np, w_np = synth.routing(2, T, E, topk)
    ids, tw = dev_i32(ids_np), dev_f32(w_np)
    W13, W13sf = _nvfp4_experts(3, E, 2 * I, H)
    W2, W2sf = _nvfp4_experts(4, E, H, I)
    gs1 = dev_f32(np.full(E, 100.0, np.float32))
    gs2 = dev_f32(np.linspace(50.0, 90.0, E).astype(np.float32))
    a1 = dev_f32(np.full(E, 1e-2, np.float32))
    a2 = dev_f32(np.linspace(1e-2, 2e-2, E).astype(np.float32))
    m13 = OQ.mxfp4_quantize(synth.bf16_normal(5, (E * 2 * I, H), 0.02))
    m2 = OQ.mxfp4_quantize(synth.bf16_normal(6, (E * H, I), 0.02))
    M13, M13sf = dev_u8(m13[0].reshape(E, 2 * I, H // 2)), dev_u8(m13[1].reshape(E, 2 * I, H // 32))
    M2, M2sf = dev_u8(m2[0].reshape(E, H, I // 2)), dev_u8(m2[1].reshape(E, H, I // 32))

    def layers():
        return (bs.nvfp4_moe_layer(x, ids, tw, W13, W13sf, W2, W2sf, gs1, a1, gs2, a2),
                bs.moe_layer(x, ids, tw, M13, M13sf, M2, M2sf))

    g, out = _capture(layers)

    def set_inputs(rep):
        x.copy_(dev_bf16(synth.bf16_normal(10 + rep, (T, H))))
        i2, w2 = synth.routing(20 + rep, T, E, topk)
        ids.copy_(dev_i32(i2))
        tw.copy_(dev_f32(w2))

    _replays_match(g, out, set_inputs, layers)


def test_fused_quantize_gemm_and_split_k_in_a_graph():
    N, K = 512, 2048
    w = synth.bf16_normal(7, (N, K), 0.02)
    bq, bsf = OQ.nvfp4_quantize(w, OQ.global_scale(w))
    B, SFB = dev_u8(bq), dev_u8(bsf)
    x1 = dev_bf16(synth.bf16_normal(8, (3, K)))          # fused kernel
    x2 = dev_bf16(synth.bf16_normal(9, (300, K)))        # quantiser + GEMM through the workspace
    gs = dev_f32(np.array([3.0], np.float32))
    a = bs.quantize(dev_bf16(synth.bf16_normal(10, (640, 7168))), "nvfp4", gs=gs)
    w2 = synth.bf16_normal(11, (1024, 7168), 0.02)
    b2q, b2sf = OQ.nvfp4_quantize(w2, OQ.global_scale(w2))
    B2, SFB2 = dev_u8(b2q), dev_u8(b2sf)

    def calls():
        return (bs.quantize_gemm(x1, gs, B, SFB), bs.quantize_gemm(x2, gs, B, SFB),
                bs.gemm(a[0], a[1], B2, SFB2))       # 640 x 1024 x 7168: split-K + reduce

    g, out = _capture(calls)

    def set_inputs(rep):
        x1.copy_(dev_bf16(synth.bf16_normal(30 + rep, (3, K))))
        x2.copy_(dev_bf16(synth.bf16_normal(40 + rep, (300, K))))
        q, sf = bs.quantize(dev_bf16(synth.bf16_normal(50 + rep, (640, 7168))), "nvfp4", gs=gs)
        a[0].copy_(q)
        a[1].copy_(sf)

    _replays_match(g, out, set_inputs, calls)

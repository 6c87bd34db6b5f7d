"""GPU parity: the fused NVFP4 quantise + GEMM (`nvfp4_quantize_gemm`).

The fused op must give, bit for bit, the output of `fp4_quantize` followed by
`fp4_gemm` (the fused kernel for up to four rows feeds the MFMA the same
exactly dequantised fp16 values in the same order; larger problems take the
two-kernel path through the workspace), and it is checked against the oracle
(oracle quantiser, float64 GEMM) with the GEMM tolerance.  Inputs: bf16
N(0,1) activations with 0.1 % outliers x20 and some all-zero and negative-zero
blocks; bf16 N(0, 0.02) weights quantised by the oracle; gs from the GPU's
global scale.
"""
import numpy as np
import pytest
import torch

import block_scaled_fp4_e2m1_amd as bs
from block_scaled_fp4_e2m1_amd import synth
from oracle import formats as F
from oracle import gemm as OG
from oracle import quant as OQ
from oracle import tolerance as TOL
from gpu_helpers import dev_bf16, dev_f32, dev_u8, host_bf16_bits

pytestmark = pytest.mark.gpu


def _problem(M, N, K, seed):
    x = synth.bf16_normal_with_outliers(seed, seed + 1, (M, K))
    x = x.copy()
    if K >= 64:
        x[0, 16:32] = 0                  # an all-zero block
        x[M - 1, 32:48] = 0x8000         # a block of negative zeros
    w = synth.bf16_normal(seed + 2, (N, K), 0.02)
    gw = OQ.global_scale(w)
    bq, sfb = OQ.nvfp4_quantize(w, gw)
    return x, bq, sfb, gw


SHAPES = [
    (1, 32, 32), (1, 7168, 7168), (2, 4096, 7168), (3, 1056, 4160), (4, 2048, 8192),
    (4, 64, 96), (1, 96, 9216),                 # K above the fused kernel's limit: two kernels
    (5, 512, 1024), (16, 4096, 7168), (64, 288, 2048), (300, 544, 1056),
]


@pytest.mark.parametrize("shape", SHAPES)
def test_quantize_gemm_equals_two_calls_and_oracle(shape):
    M, N, K = shape
    x, bq, sfb, gw = _problem(M, N, K, 7 + M + K)
    dx = dev_bf16(x)
    gs = bs.global_scale(dx)
    B, SFB = dev_u8(bq), dev_u8(sfb)
    alpha = (1.0 / (gs * torch.tensor([gw], device=gs.device))).float().contiguous()
    d_fused = bs.quantize_gemm(dx, gs, B, SFB, alpha)
    q, sf = bs.quantize(dx, "nvfp4", gs=gs)
    d_two = bs.gemm(q, sf, B, SFB, alpha)
    torch.cuda.synchronize()
    got = host_bf16_bits(d_fused)
    assert np.array_equal(got, host_bf16_bits(d_two)), shape
    g = np.float32(gs.cpu().numpy()[0])
    assert g == OQ.global_scale(x)
    xq, xsf = OQ.nvfp4_quantize(x, g)
    assert np.array_equal(q.cpu().numpy(), xq) and np.array_equal(sf.cpu().numpy(), xsf)
    ref = OG.nvfp4_gemm(xq, xsf, bq, sfb, np.float32(alpha.cpu().numpy()[0]))
    ok, worst, nbad = TOL.check_bf16(got, ref)
    assert ok, f"{shape}: {nbad} out of tolerance (worst {worst:.2f})"


def test_quantize_gemm_repeated_calls_and_saturating_scale():
    """A gs that saturates block scales (E4M3 448) and back-to-back calls on one stream."""
    M, N, K = 4, 256, 2048
    x, bq, sfb, _ = _problem(M, N, K, 99)
    dx = dev_bf16(x)
    B, SFB = dev_u8(bq), dev_u8(sfb)
    for gsv in (np.float32(1e6), np.float32(1e-3), np.float32(OQ.global_scale(x))):
        gs = dev_f32(np.array([gsv]))
        outs = [bs.quantize_gemm(dx, gs, B, SFB) for _ in range(3)]
        q, sf = bs.quantize(dx, "nvfp4", gs=gs)
        d_two = bs.gemm(q, sf, B, SFB)
        torch.cuda.synchronize()
        for o in outs:
            assert np.array_equal(host_bf16_bits(o), host_bf16_bits(d_two)), gsv

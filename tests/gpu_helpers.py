"""Shared helpers for the GPU parity tests (host <-> device marshalling)."""
import numpy as np
import torch

from block_scaled_fp4_e2m1_amd import synth
from oracle import quant as OQ

DEV = "cuda:0"


def dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


def dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(
        torch.bfloat16).to(DEV)


def host_bf16_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def nvfp4_problem(M, N, K, seed, a_std=1.0, b_std=1.0):
    """bf16 N(0, std) activations/weights quantised by the oracle recipe."""
    a = synth.bf16_normal(seed, (M, K), a_std)
    b = synth.bf16_normal(seed + 1, (N, K), b_std)
    ga, gb = OQ.global_scale(a), OQ.global_scale(b)
    aq, sfa = OQ.nvfp4_quantize(a, ga)
    bq, sfb = OQ.nvfp4_quantize(b, gb)
    alpha = np.float32(np.float32(1.0) / np.float32(ga * gb))
    return aq, sfa, bq, sfb, alpha


def mxfp4_problem(M, N, K, seed, a_std=1.0, b_std=1.0):
    a = synth.bf16_normal(seed, (M, K), a_std)
    b = synth.bf16_normal(seed + 1, (N, K), b_std)
    aq, sfa = OQ.mxfp4_quantize(a)
    bq, sfb = OQ.mxfp4_quantize(b)
    return aq, sfa, bq, sfb

"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle.

This module holds no step of the quantisers or GEMMs: it only draws random
numbers (numpy PCG64) and rounds them to bf16 with torch's float32->bf16
cast (round to nearest even).  Everything returns host numpy arrays; bf16
tensors are returned as their uint16 bit patterns.

Workload shapes follow the pages' benchmarks: activations ~ N(0, 1),
weights ~ N(0, 0.02), activations optionally carrying a small fraction of
outliers scaled by 20, and MoE routing drawn as the top-k of a softmax over
N(0, 1) logits.
"""
from __future__ import annotations

import numpy as np
import torch


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_normal(seed: int, shape, std: float = 1.0) -> np.ndarray:
    """bf16 bits of N(0, std^2) samples: float32 draw times std, then RNE to bf16."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape, dtype=np.float32) * np.float32(std)
    return f32_to_bf16_bits(x)


def bf16_normal_with_outliers(seed: int, outlier_seed: int, shape, frac: float = 0.001,
                              factor: float = 20.0) -> np.ndarray:
    """N(0,1) activations where round(frac * numel) distinct positions (drawn
    without replacement) are multiplied by `factor` in float32 before the
    bf16 rounding."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape, dtype=np.float32)
    n = int(round(frac * x.size))
    pos = np.random.default_rng(outlier_seed).choice(x.size, size=n, replace=False)
    flat = x.reshape(-1)
    flat[pos] = flat[pos] * np.float32(factor)
    return f32_to_bf16_bits(x)


def routing(seed: int, num_tokens: int, num_experts: int, topk: int):
    """(topk_ids int32 [T, topk], topk_weights float32 [T, topk]).

    Logits ~ N(0,1) in float32; probabilities = softmax in float64; the topk
    largest probabilities per token (ties to the lower expert index), their
    probabilities rounded to float32, not renormalised.
    """
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((num_tokens, num_experts), dtype=np.float32).astype(np.float64)
    z = logits - logits.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    order = np.argsort(-p, axis=1, kind="stable")[:, :topk]
    w = np.take_along_axis(p, order, axis=1).astype(np.float32)
    return order.astype(np.int32), w


def random_bytes(seed: int, shape) -> np.ndarray:
    return np.random.default_rng(seed).integers(0, 256, size=shape, dtype=np.uint8)


def random_e4m3_scales(seed: int, shape, lo: int = 0x20, hi: int = 0x48) -> np.ndarray:
    """Random finite positive E4M3 scale codes in [lo, hi)."""
    return np.random.default_rng(seed).integers(lo, hi, size=shape, dtype=np.uint8)


def random_e8m0_scales(seed: int, shape, lo: int = 120, hi: int = 134) -> np.ndarray:
    """Random E8M0 scale codes in [lo, hi) (2**-7 .. 2**6)."""
    return np.random.default_rng(seed).integers(lo, hi, size=shape, dtype=np.uint8)

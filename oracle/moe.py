"""MXFP4 and NVFP4 W4A4 mixture-of-experts layers, stage by stage (CPU oracle).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

What the pages fix:
  * "[Kernel] Enable CUTLASS MXFP4 W4A4 MoE on SM12x": activations are
    quantised to MXFP4 per expert group (`mxfp4_experts_quant`) and
    multiplied by per-expert MXFP4 weights in a grouped GEMM.
  * vLLM `sm103` branch comparison page, `csrc/ops.h` /
    `torch_bindings.cpp`: the fused `silu_and_mul_scaled_fp4_experts_quant`
    op and the per-expert quant take `input_offset_by_experts` and
    `output_scale_offset_by_experts`, i.e. rows are grouped by expert and
    addressed through per-expert offsets.

Readings where the pages are silent (listed in the design notes):
  * rows are sorted stably by expert; within an expert they keep the order
    of the flat index t * topk + j (token t, routing slot j);
  * gate = first half of the gate_up output, up = second half,
    act = bf16(silu(gate) * up) with silu(g) = g / (1 + exp(-g)) in float64
    from the bf16 gate_up output;
  * every expert GEMM has alpha = 1 (the E8M0 scales carry all scaling);
  * the combine sums w[t, j] * Y over the token's slots from the unrounded
    down-projection output Y and rounds once to bf16; weights are not
    renormalised.

NVFP4 form (the per-expert NVFP4 ops the vLLM `sm103` branch comparison page
declares: `scaled_fp4_experts_quant` and `silu_and_mul_scaled_fp4_experts_quant`,
which take per-expert offsets; their bodies are not printed).  Readings:
  * each expert e has its own activation global scales gs1[e] (input of
    gate_up) and gs2[e] (input of down) and its own FP32 GEMM alphas
    alpha1[e], alpha2[e], the dense NVFP4 conventions applied per expert;
  * a sorted row of expert e is quantised with the NVFP4 recipe of the dense
    quantiser using gs of that expert (so the same token routed to two
    experts may quantise differently and cannot be shared);
  * h1 = bf16(alpha1[e] * dec(xq) @ dec(W13[e])^T); act = bf16(silu(g) * u)
    as in the MXFP4 form; act rows are NVFP4-quantised with gs2[e];
    y = alpha2[e] * dec(aq) @ dec(W2[e])^T unrounded; the same combine.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_bits_to_f64, bf16_rne_from_f64
from .quant import mxfp4_dequantize, mxfp4_quantize, nvfp4_dequantize, nvfp4_quantize


def moe_prep(topk_ids, num_experts: int):
    """(expert_offsets int32 [E+1], sorted_ids int32 [T*topk]).

    sorted_ids[r] is the flat index t * topk + j of the r-th row in expert
    order; rows of expert e occupy [offsets[e], offsets[e+1]).
    """
    ids = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    if ids.size and (ids.min() < 0 or ids.max() >= num_experts):
        raise ValueError("expert id out of range")
    counts = np.bincount(ids, minlength=num_experts)
    offsets = np.zeros(num_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    order = np.argsort(ids, kind="stable")
    return offsets.astype(np.int32), order.astype(np.int32)


def experts_quant(x_bf16_bits, sorted_ids, topk: int):
    """MXFP4 codes and scales of x[token of sorted row r] for every sorted row."""
    x = np.asarray(x_bf16_bits, dtype=np.uint16)
    tokens = np.asarray(sorted_ids, dtype=np.int64) // topk
    return mxfp4_quantize(x[tokens])


def grouped_gemm_f64(Aq, Asf, offsets, Wq, Wsf) -> np.ndarray:
    """Per expert e: rows [offsets[e], offsets[e+1]) of dequant(A) @ dequant(W[e])^T."""
    offsets = np.asarray(offsets, dtype=np.int64)
    E = offsets.size - 1
    R = int(offsets[-1])
    N = Wq.shape[1]
    out = np.zeros((R, N), dtype=np.float64)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        a = mxfp4_dequantize(Aq[lo:hi], Asf[lo:hi])
        w = mxfp4_dequantize(Wq[e], Wsf[e])
        out[lo:hi] = a @ w.T
    return out


def silu_mul(h_bf16_bits) -> np.ndarray:
    """act = bf16(silu(g) * u), g = first half of the columns, u = second half."""
    h = bf16_bits_to_f64(h_bf16_bits)
    inter = h.shape[1] // 2
    g = h[:, :inter]
    u = h[:, inter:]
    return bf16_rne_from_f64(g / (1.0 + np.exp(-g)) * u)


def combine(Y, sorted_ids, topk_weights, num_tokens: int) -> np.ndarray:
    """out[t] = bf16(sum_j w[t, j] * Y[row of (t, j)]), summed in float64."""
    Y = np.asarray(Y, dtype=np.float64)
    w = np.asarray(topk_weights, dtype=np.float32).reshape(-1).astype(np.float64)
    flat = np.asarray(sorted_ids, dtype=np.int64)
    acc = np.zeros((num_tokens, Y.shape[1]), dtype=np.float64)
    np.add.at(acc, flat // (w.size // num_tokens), w[flat][:, None] * Y)
    return bf16_rne_from_f64(acc)


def moe_layer(x_bf16_bits, topk_ids, topk_weights, W13q, W13sf, W2q, W2sf):
    """The whole layer from scratch; returns every intermediate stage.

    Stage names: offsets, sorted_ids, xq, xsf, h1 (bf16), act (bf16),
    aq, asf, y (float64, unrounded), out (bf16).
    """
    T, topk = np.asarray(topk_ids).shape
    E = W13q.shape[0]
    offsets, sorted_ids = moe_prep(topk_ids, E)
    xq, xsf = experts_quant(x_bf16_bits, sorted_ids, topk)
    h1 = bf16_rne_from_f64(grouped_gemm_f64(xq, xsf, offsets, W13q, W13sf))
    act = silu_mul(h1)
    aq, asf = mxfp4_quantize(act)
    y = grouped_gemm_f64(aq, asf, offsets, W2q, W2sf)
    out = combine(y, sorted_ids, topk_weights, T)
    return dict(offsets=offsets, sorted_ids=sorted_ids, xq=xq, xsf=xsf, h1=h1,
                act=act, aq=aq, asf=asf, y=y, out=out)


def _expert_ranges(offsets):
    offsets = np.asarray(offsets, dtype=np.int64)
    for e in range(offsets.size - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            yield e, lo, hi


def nvfp4_rows_quant(x_bf16_bits, offsets, gs_experts):
    """NVFP4 codes and scales of sorted rows x[r], row r of expert e with gs_experts[e]."""
    x = np.asarray(x_bf16_bits, dtype=np.uint16)
    R, K = x.shape
    gs = np.asarray(gs_experts, dtype=np.float32)
    q = np.zeros((R, K // 2), dtype=np.uint8)
    sf = np.zeros((R, K // 16), dtype=np.uint8)
    for e, lo, hi in _expert_ranges(offsets):
        q[lo:hi], sf[lo:hi] = nvfp4_quantize(x[lo:hi], gs[e])
    return q, sf


def nvfp4_experts_quant(x_bf16_bits, sorted_ids, topk: int, offsets, gs_experts):
    """Sorted row r = x[token of r] quantised with the global scale of r's expert."""
    x = np.asarray(x_bf16_bits, dtype=np.uint16)
    tokens = np.asarray(sorted_ids, dtype=np.int64) // topk
    return nvfp4_rows_quant(x[tokens], offsets, gs_experts)


def nvfp4_grouped_gemm_f64(Aq, Asf, offsets, Wq, Wsf, alphas) -> np.ndarray:
    """Per expert e: alpha[e] * dec(A rows of e) @ dec(W[e])^T, unrounded."""
    offsets = np.asarray(offsets, dtype=np.int64)
    al = np.asarray(alphas, dtype=np.float32).astype(np.float64)
    out = np.zeros((int(offsets[-1]), Wq.shape[1]), dtype=np.float64)
    for e, lo, hi in _expert_ranges(offsets):
        out[lo:hi] = al[e] * (nvfp4_dequantize(Aq[lo:hi], Asf[lo:hi]) @ nvfp4_dequantize(Wq[e], Wsf[e]).T)
    return out


def nvfp4_moe_layer(x_bf16_bits, topk_ids, topk_weights, W13q, W13sf, W2q, W2sf, gs1, alpha1, gs2,
                    alpha2):
    """The NVFP4 layer from scratch; the same stage names as moe_layer."""
    T, topk = np.asarray(topk_ids).shape
    E = W13q.shape[0]
    offsets, sorted_ids = moe_prep(topk_ids, E)
    xq, xsf = nvfp4_experts_quant(x_bf16_bits, sorted_ids, topk, offsets, gs1)
    h1 = bf16_rne_from_f64(nvfp4_grouped_gemm_f64(xq, xsf, offsets, W13q, W13sf, alpha1))
    act = silu_mul(h1)
    aq, asf = nvfp4_rows_quant(act, offsets, gs2)
    y = nvfp4_grouped_gemm_f64(aq, asf, offsets, W2q, W2sf, alpha2)
    out = combine(y, sorted_ids, topk_weights, T)
    return dict(offsets=offsets, sorted_ids=sorted_ids, xq=xq, xsf=xsf, h1=h1,
                act=act, aq=aq, asf=asf, y=y, out=out)

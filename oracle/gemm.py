"""Block-scaled FP4 GEMMs as their plain definition, in float64 (CPU oracle).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

What the pages fix:
  * vLLM `sm103` branch comparison page, `nvfp4_scaled_mm_kernels.cu`
    (`Fp4GemmSm103`, `cutlass_scaled_fp4_mm_sm103a_impl`): A is [M, K/2]
    packed E2M1 (row-major, K contiguous), B is [N, K/2] packed E2M1 (each
    output column's weights contiguous along K), one E4M3 scale per 16
    K-elements for each operand, an FP32 `alpha`, FP32 accumulation, and a
    bf16 (or fp16) D = [M, N].
  * "perf(gemm): optimize SM103 CuTe DSL mm_fp4 kernel", section "Alpha
    epilogue bug": alpha multiplies the FP32 accumulator, followed by one
    conversion to the output type.
  * "feat: sm100 cute_dsl w4a16 gemm" (follow-up PR body, "Description"):
    W4A16 multiplies bf16 activations by NVFP4 weights, and the one FP32
    scale of the whole weight tensor multiplies the FP32 sums before the
    output conversion.
  * "[Kernel] Enable CUTLASS MXFP4 W4A4 MoE on SM12x": MXFP4 x MXFP4 GEMM
    with E8M0 scales per 32 elements.

The method reaches the plain result D = bf16(alpha * dequant(A) @
dequant(B)^T) up to FP32 summation order, so the oracle computes exactly
that: every operand is decoded to float64 (exact: at most 6 significant
bits per product factor), one float64 matrix product (a library step),
one multiplication by alpha, and one round-to-nearest-even to bf16.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_bits_to_f64, bf16_rne_from_f64
from .quant import mxfp4_dequantize, nvfp4_dequantize


def _check_k(a_cols: int, b_cols: int):
    if a_cols != b_cols:
        raise ValueError("A and B disagree on K")


def nvfp4_gemm_f64(Aq, SFA, Bq, SFB, alpha) -> np.ndarray:
    """Unrounded float64 alpha * sum_k dec(A)[m,k] * dec(B)[n,k]."""
    a = nvfp4_dequantize(Aq, SFA)
    b = nvfp4_dequantize(Bq, SFB)
    _check_k(a.shape[1], b.shape[1])
    return np.float64(np.float32(alpha)) * (a @ b.T)


def mxfp4_gemm_f64(Aq, SFA, Bq, SFB, alpha=1.0) -> np.ndarray:
    a = mxfp4_dequantize(Aq, SFA)
    b = mxfp4_dequantize(Bq, SFB)
    _check_k(a.shape[1], b.shape[1])
    return np.float64(np.float32(alpha)) * (a @ b.T)


def w4a16_gemm_f64(A_bf16_bits, Bq, SFB, alpha) -> np.ndarray:
    a = bf16_bits_to_f64(A_bf16_bits)
    b = nvfp4_dequantize(Bq, SFB)
    _check_k(a.shape[1], b.shape[1])
    return np.float64(np.float32(alpha)) * (a @ b.T)


def nvfp4_gemm(Aq, SFA, Bq, SFB, alpha) -> np.ndarray:
    """bf16 bit patterns (uint16 [M, N]) of the NVFP4 W4A4 GEMM."""
    return bf16_rne_from_f64(nvfp4_gemm_f64(Aq, SFA, Bq, SFB, alpha))


def mxfp4_gemm(Aq, SFA, Bq, SFB, alpha=1.0) -> np.ndarray:
    """bf16 bit patterns (uint16 [M, N]) of the MXFP4 W4A4 GEMM."""
    return bf16_rne_from_f64(mxfp4_gemm_f64(Aq, SFA, Bq, SFB, alpha))


def w4a16_gemm(A_bf16_bits, Bq, SFB, alpha) -> np.ndarray:
    """bf16 bit patterns (uint16 [M, N]) of the bf16 x NVFP4 GEMM."""
    return bf16_rne_from_f64(w4a16_gemm_f64(A_bf16_bits, Bq, SFB, alpha))

"""NVFP4 and MXFP4 block quantisers and dequantisers (CPU oracle).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

What the pages fix:
  * vLLM `sm103` branch comparison page, `nvfp4_quant_kernels.cu`,
    `cvt_fp16_to_fp4_sm103`: bf16 rows are quantised in 16-element blocks
    along the row, one scale byte per block, two E2M1 codes per output
    byte with the earlier element in the low bits; with `UE8M0_SF` the
    scale is a power of two.  The per-block routine it calls
    (`cvt_warp_fp16_to_fp4`) is not printed.
  * same page, `test_nvfp4_quant.py`
    (`test_scaled_fp4_quant_sm103_matches_sm100`): the tensor-wide global
    scale is FLOAT8_E4M3_MAX * FLOAT4_E2M1_MAX / amax(|x|) = 2688 / amax.
  * "[Kernel] Enable CUTLASS MXFP4 W4A4 MoE on SM12x" page: MXFP4
    activations are quantised per expert group (`mxfp4_experts_quant`);
    the MX form carries its scale in an E8M0 byte per 32 elements.

Readings where the pages are silent (each listed in the design notes):
  * NVFP4 block scale s = fl32(fl32(amax / 6) * gs), rounded to E4M3 by
    round-to-nearest-even with saturation at 448.
  * value multiplier inv = fl32(gs / decode(sf)), or 0 when the scale
    decodes to 0; codes = E2M1-RNE(fl32(v * inv)), keeping the sign bit.
  * MXFP4 block scale = the smallest power of two >= fl32(amax / 6), so no
    element saturates; inv = 2**(127 - sf) exactly.
"""
from __future__ import annotations

import numpy as np

from .formats import (
    E2M1_TABLE,
    E4M3_TABLE,
    E8M0_TABLE,
    bf16_bits_to_f32,
    e2m1_encode,
    e4m3_encode_satfinite,
    e8m0_encode_ceil,
    pack_nibbles,
    unpack_nibbles,
)

NVFP4_BLOCK = 16
MXFP4_BLOCK = 32


def global_scale(x_bf16_bits) -> np.float32:
    """gs = fl32(2688 / amax(|x|)) over the whole tensor, all in binary32."""
    v = bf16_bits_to_f32(x_bf16_bits)
    amax = np.max(np.abs(v))
    return np.float32(np.float32(448.0 * 6.0) / amax)


def nvfp4_quantize(x_bf16_bits, gs):
    """Quantise bf16 rows [R, K] (uint16 bit patterns) to NVFP4.

    Returns (q uint8 [R, K/2], sf uint8 [R, K/16]) in row-major order.
    For each row and each 16-element block along K:
      1. v_i   = the block's elements widened to binary32 (exact)
      2. amax  = max_i |v_i|
      3. s     = fl32(fl32(amax / 6) * gs)
      4. sf    = E4M3 code of s (RNE, saturating at 448); sdec = its value
      5. inv   = fl32(gs / sdec), or 0 if sdec == 0
      6. code  = E2M1-RNE(fl32(v_i * inv))
    """
    v = bf16_bits_to_f32(x_bf16_bits)
    if v.ndim != 2 or v.shape[1] % NVFP4_BLOCK:
        raise ValueError("nvfp4_quantize expects [R, K] with K % 16 == 0")
    gs = np.float32(gs)
    R, K = v.shape
    blocks = v.reshape(R, K // NVFP4_BLOCK, NVFP4_BLOCK)
    amax = np.max(np.abs(blocks), axis=2)                       # float32
    with np.errstate(over="ignore"):                            # overflow to inf saturates below
        s = (amax / np.float32(6.0)) * gs                       # two fp32 roundings
    sf = e4m3_encode_satfinite(s)
    sdec = E4M3_TABLE[sf].astype(np.float32)                    # exact
    with np.errstate(divide="ignore"):
        inv = np.where(sdec == 0, np.float32(0.0), gs / sdec).astype(np.float32)
    with np.errstate(over="ignore"):                            # +-inf encodes as +-6
        y = blocks * inv[:, :, None]                            # fp32 multiply
    codes = e2m1_encode(y).reshape(R, K)
    return pack_nibbles(codes), sf


def mxfp4_quantize(x_bf16_bits):
    """Quantise bf16 rows [R, K] (uint16 bit patterns) to MXFP4.

    Returns (q uint8 [R, K/2], sf uint8 [R, K/32]).  For each 32-block:
      1. amax = max |v_i|
      2. sf   = E8M0 code of the smallest power of two >= fl32(amax / 6)
      3. inv  = 2**(127 - sf)   (exact in binary32 for sf in [0, 254])
      4. code = E2M1-RNE(fl32(v_i * inv))
    """
    v = bf16_bits_to_f32(x_bf16_bits)
    if v.ndim != 2 or v.shape[1] % MXFP4_BLOCK:
        raise ValueError("mxfp4_quantize expects [R, K] with K % 32 == 0")
    R, K = v.shape
    blocks = v.reshape(R, K // MXFP4_BLOCK, MXFP4_BLOCK)
    amax = np.max(np.abs(blocks), axis=2)
    s = amax / np.float32(6.0)
    sf = e8m0_encode_ceil(s)
    inv = np.ldexp(np.float32(1.0), 127 - sf.astype(np.int32)).astype(np.float32)
    y = blocks * inv[:, :, None]
    codes = e2m1_encode(y).reshape(R, K)
    return pack_nibbles(codes), sf


def nvfp4_dequantize(q, sf) -> np.ndarray:
    """Exact float64 values e2m1(code) * e4m3(scale) of NVFP4 rows [R, K]."""
    codes = unpack_nibbles(q)
    scale = np.repeat(E4M3_TABLE[np.asarray(sf, dtype=np.uint8)], NVFP4_BLOCK, axis=-1)
    return E2M1_TABLE[codes] * scale


def mxfp4_dequantize(q, sf) -> np.ndarray:
    """Exact float64 values e2m1(code) * 2**(scale-127) of MXFP4 rows [R, K]."""
    codes = unpack_nibbles(q)
    scale = np.repeat(E8M0_TABLE[np.asarray(sf, dtype=np.uint8)], MXFP4_BLOCK, axis=-1)
    return E2M1_TABLE[codes] * scale

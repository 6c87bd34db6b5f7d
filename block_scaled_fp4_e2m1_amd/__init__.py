"""Block-scaled FP4 (E2M1) GEMMs for AMD Instinct MI355X (gfx950).

The computation lives in libbsfp4.so (hand-written HIP kernels behind a C
ABI, declared in include/bsfp4.h); `binding` marshals torch tensors into it.
"""
from .binding import (  # noqa: F401
    MOE_SILU_MUL_QUANT,
    MOE_STORE_BF16,
    MOE_WEIGHTED_COMBINE,
    MXFP4,
    NVFP4,
    SF_LAYOUTS,
    Bsfp4Error,
    e2m1_convert,
    global_scale,
    gemm,
    load,
    moe_layer,
    moe_prep,
    mxfp4_moe_grouped_gemm,
    nvfp4_experts_quantize,
    nvfp4_moe_grouped_gemm,
    nvfp4_moe_layer,
    quantize,
    quantize_gemm,
    scales_swizzle,
    scales_unswizzle,
    version,
    w4a16_gemm,
)

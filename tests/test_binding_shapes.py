"""CPU checks of the Python binding's extent validation.

The C ABI receives raw pointers, so the binding must refuse every tensor whose
extent does not match the call (an undersized scale or output tensor would
otherwise become an out-of-bounds device access).  These tests use meta
tensors: a correctly shaped call gets through every shape check and stops at
the device check ("must be a device tensor"); each wrong extent is refused with
its own message before that.  Nothing here touches a GPU or the library.
"""
import pytest
import torch

import block_scaled_fp4_e2m1_amd as bs

U8, BF16, F32, I32 = torch.uint8, torch.bfloat16, torch.float32, torch.int32


def m(*shape, dtype=U8):
    return torch.empty(shape, dtype=dtype, device="meta")


def reaches_device_check(fn, *a, **kw):
    with pytest.raises(ValueError, match="must be a device tensor"):
        fn(*a, **kw)


def refused(match, fn, *a, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*a, **kw)


def test_gemm_extents():
    M, N, K = 16, 64, 256
    A, SFA, B, SFB = m(M, K // 2), m(M, K // 16), m(N, K // 2), m(N, K // 16)
    al = m(1, dtype=F32)
    reaches_device_check(bs.gemm, A, SFA, B, SFB, al)
    reaches_device_check(bs.gemm, A, SFA, B, SFB, al, out=m(M, N, dtype=BF16))
    refused("B has K", bs.gemm, A, SFA, m(N, K // 2 - 16), SFB, al)
    refused("SFA must hold", bs.gemm, A, m(M, K // 16 - 1), B, SFB, al)
    refused("SFB must hold", bs.gemm, A, SFA, B, m(N - 1, K // 16), al)
    refused("out must have shape", bs.gemm, A, SFA, B, SFB, al, out=m(M, N - 32, dtype=BF16))
    refused("out must have shape", bs.gemm, A, SFA, B, SFB, al, out=m(M + 1, N, dtype=BF16))
    refused("alpha must hold", bs.gemm, A, SFA, B, SFB, m(2, dtype=F32))
    refused("A must be 2-D", bs.gemm, m(M, K // 2, 1), SFA, B, SFB, al)
    # NVFP4 scales passed to the MXFP4 form: twice too many bytes
    refused("SFA must hold", bs.gemm, A, SFA, B, m(N, K // 32), None, fmt="mxfp4")
    reaches_device_check(bs.gemm, A, m(M, K // 32), B, m(N, K // 32), None, fmt="mxfp4")
    with pytest.raises(TypeError):
        bs.gemm(A, SFA, B, SFB, m(1, dtype=BF16))


def test_quantize_extents():
    x = m(8, 64, dtype=BF16)
    gs = m(1, dtype=F32)
    reaches_device_check(bs.quantize, x, "nvfp4", gs=gs)
    reaches_device_check(bs.quantize, x, "mxfp4")
    refused("needs the global scale", bs.quantize, x, "nvfp4")
    refused("takes no global scale", bs.quantize, x, "mxfp4", gs=gs)
    refused("multiple of 32", bs.quantize, m(8, 48, dtype=BF16), "mxfp4")
    refused("q must have shape", bs.quantize, x, "nvfp4", gs=gs, q=m(8, 31))
    refused("sf must hold", bs.quantize, x, "nvfp4", gs=gs, sf=m(8, 2))
    rm = m(5, dtype=I32)
    reaches_device_check(bs.quantize, x, "mxfp4", row_map=rm, q=m(5, 32), sf=m(5, 2))
    refused("q must have shape", bs.quantize, x, "mxfp4", row_map=rm, q=m(8, 32))
    refused("gs must hold", bs.quantize, x, "nvfp4", gs=m(2, dtype=F32))


def test_w4a16_and_quantize_gemm_extents():
    M, N, K = 4, 64, 256
    A, B, SFB = m(M, K, dtype=BF16), m(N, K // 2), m(N, K // 16)
    reaches_device_check(bs.w4a16_gemm, A, B, SFB, m(1, dtype=F32))
    refused("B has K", bs.w4a16_gemm, A, m(N, K // 4), SFB)
    refused("SFB must hold", bs.w4a16_gemm, A, B, m(N, K // 32))
    refused("out must have shape", bs.w4a16_gemm, A, B, SFB, out=m(M, N // 2, dtype=BF16))
    gs = m(1, dtype=F32)
    reaches_device_check(bs.quantize_gemm, A, gs, B, SFB)
    refused("x has K", bs.quantize_gemm, A, gs, m(N, K), SFB)
    refused("SFB must hold", bs.quantize_gemm, A, gs, B, m(N, 1))
    refused("gs must hold", bs.quantize_gemm, A, m(3, dtype=F32), B, SFB)
    refused("out must have shape", bs.quantize_gemm, A, gs, B, SFB, out=m(M, N, 1, dtype=BF16))


def test_scale_layout_extents():
    reaches_device_check(bs.scales_swizzle, m(200, 13))
    refused("out must hold", bs.scales_swizzle, m(200, 13), out=m(200, 16))
    reaches_device_check(bs.scales_unswizzle, m(256, 16), 200, 13)
    refused("swz must hold", bs.scales_unswizzle, m(200, 13), 200, 13)
    refused("out must hold", bs.scales_unswizzle, m(256, 16), 200, 13, out=m(200, 12))


def test_mxfp4_grouped_extents():
    E, N, K, rows = 4, 128, 256, 40
    Aq, Asf = m(rows, K // 2), m(rows, K // 32)
    W, Wsf, offs = m(E, N, K // 2), m(E, N, K // 32), m(E + 1, dtype=I32)
    G = bs.mxfp4_moe_grouped_gemm
    reaches_device_check(G, Aq, Asf, offs, W, Wsf)
    refused("W has K", G, Aq, Asf, offs, m(E, N, K // 4), Wsf)
    refused("Wsf must hold", G, Aq, Asf, offs, W, m(E, N, K // 16))
    refused("Asf must hold", G, Aq, m(rows, K // 16), offs, W, Wsf)
    refused("expert_offsets must hold", G, Aq, Asf, m(E, dtype=I32), W, Wsf)
    refused("W must be 3-D", G, Aq, Asf, offs, m(E * N, K // 2), Wsf)
    refused("out must have shape", G, Aq, Asf, offs, W, Wsf, out=m(rows - 1, N, dtype=BF16))
    # gather form: rows follow the index, Aq may hold fewer (token) rows
    idx = m(rows, dtype=I32)
    reaches_device_check(G, m(10, K // 2), m(10, K // 32), offs, W, Wsf, a_row_index=idx)
    refused("exceeds len", G, m(10, K // 2), m(10, K // 32), offs, W, Wsf, a_row_index=idx, rows=rows + 1)
    refused("must equal Aq.shape", G, Aq, Asf, offs, W, Wsf, rows=rows - 1)
    # SiLU-mul + re-quant outputs: act width N/2, one E8M0 byte per 32 act values
    S = bs.MOE_SILU_MUL_QUANT
    reaches_device_check(G, Aq, Asf, offs, W, Wsf, S, out_q=m(rows, N // 4), out_sf=m(rows, N // 64))
    refused("out_q must have shape", G, Aq, Asf, offs, W, Wsf, S, out_q=m(rows, N // 2))
    refused("out_sf must hold", G, Aq, Asf, offs, W, Wsf, S, out_sf=m(rows, N // 32))
    refused("N % 64", G, Aq, Asf, offs, m(E, 96, K // 2), m(E, 96, K // 32), S)
    # combine: rows = tokens x topk, per-row ids and weights, [T, N] output
    C = bs.MOE_WEIGHTED_COMBINE
    ids, w = m(rows, dtype=I32), m(rows, dtype=F32)
    reaches_device_check(G, Aq, Asf, offs, W, Wsf, C, sorted_ids=ids, topk_weights=w, num_tokens=10, topk=4)
    refused("num_tokens \\* topk == rows", G, Aq, Asf, offs, W, Wsf, C, sorted_ids=ids, topk_weights=w,
            num_tokens=10, topk=3)
    refused("needs sorted_ids", G, Aq, Asf, offs, W, Wsf, C, topk_weights=w, num_tokens=10, topk=4)
    refused("topk_weights must hold", G, Aq, Asf, offs, W, Wsf, C, sorted_ids=ids,
            topk_weights=m(rows - 4, dtype=F32), num_tokens=10, topk=4)
    refused("out must have shape", G, Aq, Asf, offs, W, Wsf, C, sorted_ids=ids, topk_weights=w,
            num_tokens=10, topk=4, out=m(rows, N, dtype=BF16))


def test_nvfp4_grouped_and_experts_quant_extents():
    E, N, K, rows = 4, 128, 256, 40
    Aq, Asf = m(rows, K // 2), m(rows, K // 16)
    W, Wsf, offs = m(E, N, K // 2), m(E, N, K // 16), m(E + 1, dtype=I32)
    al = m(E, dtype=F32)
    G = bs.nvfp4_moe_grouped_gemm
    reaches_device_check(G, Aq, Asf, offs, W, Wsf, al)
    refused("alpha_experts must hold", G, Aq, Asf, offs, W, Wsf, m(E - 1, dtype=F32))
    refused("Wsf must hold", G, Aq, Asf, offs, W, m(E, N, K // 32), al)
    refused("needs out_gs", G, Aq, Asf, offs, W, Wsf, al, bs.MOE_SILU_MUL_QUANT)
    refused("out_gs must hold", G, Aq, Asf, offs, W, Wsf, al, bs.MOE_SILU_MUL_QUANT, out_gs=m(1, dtype=F32))
    reaches_device_check(G, Aq, Asf, offs, W, Wsf, al, bs.MOE_SILU_MUL_QUANT, out_gs=m(E, dtype=F32),
                         out_sf=m(rows, N // 32))
    refused("out_sf must hold", G, Aq, Asf, offs, W, Wsf, al, bs.MOE_SILU_MUL_QUANT, out_gs=m(E, dtype=F32),
            out_sf=m(rows, N // 64))
    Q = bs.nvfp4_experts_quantize
    x = m(10, K, dtype=BF16)
    reaches_device_check(Q, x, offs, m(E, dtype=F32), row_map=m(rows, dtype=I32))
    refused("gs_experts must hold", Q, x, offs, m(E + 1, dtype=F32))
    refused("q must have shape", Q, x, offs, m(E, dtype=F32), q=m(10, K // 4))
    refused("multiple of 16", Q, m(10, 40, dtype=BF16), offs, m(E, dtype=F32))


def test_moe_layer_extents():
    T, H, I, E, topk = 16, 256, 128, 4, 2
    x, ids, w = m(T, H, dtype=BF16), m(T, topk, dtype=I32), m(T, topk, dtype=F32)
    W13, W13sf = m(E, 2 * I, H // 2), m(E, 2 * I, H // 32)
    W2, W2sf = m(E, H, I // 2), m(E, H, I // 32)
    reaches_device_check(bs.moe_layer, x, ids, w, W13, W13sf, W2, W2sf)
    refused("W2 must have shape", bs.moe_layer, x, ids, w, W13, W13sf, m(E, H, I // 4), W2sf)
    refused("topk_weights must have shape", bs.moe_layer, x, ids, m(T, topk + 1, dtype=F32), W13, W13sf,
            W2, W2sf)
    refused("x has 16 tokens", bs.moe_layer, x, m(T + 1, topk, dtype=I32), m(T + 1, topk, dtype=F32), W13,
            W13sf, W2, W2sf)
    refused("W13 has K", bs.moe_layer, m(T, 2 * H, dtype=BF16), ids, w, W13, W13sf, W2, W2sf)


def test_moe_prep_extents():
    reaches_device_check(bs.moe_prep, m(16, 2, dtype=I32), 8)
    refused("must be 2-D", bs.moe_prep, m(32, dtype=I32), 8)
    refused("num_experts must be", bs.moe_prep, m(16, 2, dtype=I32), 0)


def test_mixed_devices_are_refused():
    M, N, K = 16, 64, 256
    with pytest.raises(ValueError, match="device tensor"):
        bs.gemm(torch.empty((M, K // 2), dtype=U8), m(M, K // 16), m(N, K // 2), m(N, K // 16))

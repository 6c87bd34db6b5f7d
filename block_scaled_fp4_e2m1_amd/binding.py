"""Thin Python binding of libbsfp4 (ctypes).

Argument marshalling only: each function checks dtypes/contiguity so that
it can hand raw device pointers to the C ABI, allocates outputs and
workspace with torch (device memory and streams are all torch is used for),
and calls the library on the current HIP stream.  Every step of the
computation runs in the library's gfx950 kernels; if the library is not
built, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libbsfp4.so")

NVFP4 = 0
MXFP4 = 1
_FORMATS = {"nvfp4": NVFP4, "mxfp4": MXFP4, NVFP4: NVFP4, MXFP4: MXFP4}

MOE_STORE_BF16 = 0
MOE_SILU_MUL_QUANT = 1
MOE_WEIGHTED_COMBINE = 2

_c_i64 = ctypes.c_int64
_c_ptr = ctypes.c_void_p
_c_size = ctypes.c_size_t


class MoeEpilogueArgs(ctypes.Structure):
    _fields_ = [
        ("out", _c_ptr),
        ("out_q", _c_ptr),
        ("out_sf", _c_ptr),
        ("sorted_ids", _c_ptr),
        ("topk_weights", _c_ptr),
        ("num_tokens", _c_i64),
        ("topk", _c_i64),
        ("out_gs", _c_ptr),
    ]


# name -> (restype, argtypes)
_SIGNATURES = {
    "bsfp4_version": (ctypes.c_int, []),
    "bsfp4_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "bsfp4_last_error": (ctypes.c_char_p, []),
    "fp4_global_scale_workspace_size": (_c_size, [_c_i64]),
    "fp4_global_scale": (ctypes.c_int, [_c_ptr, _c_i64, _c_ptr, _c_ptr, _c_size, _c_ptr]),
    "fp4_quantize": (ctypes.c_int, [ctypes.c_int, _c_ptr, _c_i64, _c_i64, _c_ptr, _c_ptr, _c_i64,
                                    _c_ptr, _c_ptr, _c_ptr]),
    "fp4_gemm_workspace_size": (_c_size, [ctypes.c_int, _c_i64, _c_i64, _c_i64]),
    "fp4_gemm": (ctypes.c_int, [ctypes.c_int, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr,
                                _c_i64, _c_i64, _c_i64, _c_ptr, _c_size, _c_ptr]),
    "w4a16_gemm_workspace_size": (_c_size, [_c_i64, _c_i64, _c_i64]),
    "w4a16_gemm": (ctypes.c_int, [_c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_i64, _c_i64, _c_i64,
                                  _c_ptr, _c_size, _c_ptr]),
    "fp4_scales_swizzled_size": (_c_size, [_c_i64, _c_i64]),
    "fp4_scales_swizzle": (ctypes.c_int, [ctypes.c_int, _c_ptr, _c_i64, _c_i64, _c_ptr, _c_ptr]),
    "fp4_scales_unswizzle": (ctypes.c_int, [ctypes.c_int, _c_ptr, _c_i64, _c_i64, _c_ptr, _c_ptr]),
    "fp4_moe_prep_workspace_size": (_c_size, [_c_i64, _c_i64, _c_i64]),
    "fp4_moe_prep": (ctypes.c_int, [_c_ptr, _c_i64, _c_i64, _c_i64, _c_ptr, _c_ptr, _c_ptr, _c_ptr,
                                    _c_size, _c_ptr]),
    "mxfp4_moe_grouped_gemm_workspace_size": (_c_size, [_c_i64, _c_i64, _c_i64, _c_i64, ctypes.c_int,
                                                        _c_i64]),
    "mxfp4_moe_grouped_gemm": (ctypes.c_int, [_c_ptr, _c_ptr, _c_i64, _c_ptr, _c_ptr, _c_i64, _c_i64,
                                              _c_ptr, _c_ptr, _c_i64, _c_i64, ctypes.c_int,
                                              ctypes.POINTER(MoeEpilogueArgs), _c_ptr, _c_size,
                                              _c_ptr]),
    "nvfp4_quantize_gemm_workspace_size": (_c_size, [_c_i64, _c_i64, _c_i64]),
    "nvfp4_quantize_gemm": (ctypes.c_int, [_c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_i64, _c_i64,
                                           _c_i64, _c_ptr, _c_size, _c_ptr]),
    "nvfp4_experts_quantize": (ctypes.c_int, [_c_ptr, _c_i64, _c_i64, _c_ptr, _c_ptr, _c_i64, _c_ptr,
                                              _c_i64, _c_ptr, _c_ptr, _c_ptr]),
    "nvfp4_moe_grouped_gemm_workspace_size": (_c_size, [_c_i64, _c_i64, _c_i64, _c_i64, ctypes.c_int,
                                                        _c_i64]),
    "nvfp4_moe_grouped_gemm": (ctypes.c_int, [_c_ptr, _c_ptr, _c_ptr, _c_i64, _c_i64, _c_ptr, _c_ptr,
                                              _c_ptr, _c_i64, _c_i64, ctypes.c_int,
                                              ctypes.POINTER(MoeEpilogueArgs), _c_ptr, _c_size, _c_ptr]),
}

_lib = None


def load() -> ctypes.CDLL:
    """Load libbsfp4.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m block_scaled_fp4_e2m1_amd.build` (hipcc, gfx950)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name, None)
            if fn is None:
                continue  # calling it raises AttributeError
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


class Bsfp4Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status


def _check(status: int, what: str):
    if status != 0:
        lib = load()
        msg = lib.bsfp4_last_error().decode() or lib.bsfp4_status_string(status).decode()
        raise Bsfp4Error(status, f"{what}: {msg}")


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, dtype, name):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")


def _workspace(nbytes: int, device):
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _fmt(fmt) -> int:
    try:
        return _FORMATS[fmt]
    except KeyError:
        raise ValueError(f"unknown format {fmt!r}") from None


# --------------------------------------------------------------------------- API

def version() -> int:
    return load().bsfp4_version()


def global_scale(x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Device float32[1] holding 2688 / max|x| for a bf16 tensor."""
    _need(x, torch.bfloat16, "x")
    lib = load()
    gs = out if out is not None else torch.empty(1, dtype=torch.float32, device=x.device)
    ws = _workspace(lib.fp4_global_scale_workspace_size(x.numel()), x.device)
    _check(lib.fp4_global_scale(_p(x), x.numel(), _p(gs), _p(ws), 0 if ws is None else ws.numel(),
                                _stream(x.device)), "fp4_global_scale")
    return gs


def quantize(x: torch.Tensor, fmt="nvfp4", gs: torch.Tensor | None = None,
             row_map: torch.Tensor | None = None, q: torch.Tensor | None = None,
             sf: torch.Tensor | None = None):
    """bf16 [R, K] -> (codes uint8 [R', K/2], scales uint8 [R', K/16 or K/32]).

    R' = len(row_map) when row_map is given (row r quantises x[row_map[r]]).
    """
    f = _fmt(fmt)
    _need(x, torch.bfloat16, "x")
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    R, K = x.shape
    if row_map is not None:
        _need(row_map, torch.int32, "row_map")
        rows_out = row_map.numel()
    else:
        rows_out = R
    blk = 16 if f == NVFP4 else 32
    if q is None:
        q = torch.empty((rows_out, K // 2), dtype=torch.uint8, device=x.device)
    if sf is None:
        sf = torch.empty((rows_out, K // blk), dtype=torch.uint8, device=x.device)
    if gs is not None:
        _need(gs, torch.float32, "gs")
    lib = load()
    _check(lib.fp4_quantize(f, _p(x), R, K, _p(gs), _p(row_map), rows_out, _p(q), _p(sf),
                            _stream(x.device)), "fp4_quantize")
    return q, sf


def gemm(A, SFA, B, SFB, alpha: torch.Tensor | None = None, fmt="nvfp4",
         out: torch.Tensor | None = None) -> torch.Tensor:
    """D = bf16(alpha * dequant(A) @ dequant(B)^T); A [M, K/2], B [N, K/2]."""
    f = _fmt(fmt)
    for t, n in ((A, "A"), (SFA, "SFA"), (B, "B"), (SFB, "SFB")):
        _need(t, torch.uint8, n)
    M, K = A.shape[0], A.shape[1] * 2
    N = B.shape[0]
    if alpha is not None:
        _need(alpha, torch.float32, "alpha")
    D = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    _need(D, torch.bfloat16, "out")
    lib = load()
    ws = _workspace(lib.fp4_gemm_workspace_size(f, M, N, K), A.device)
    _check(lib.fp4_gemm(f, _p(A), _p(SFA), _p(B), _p(SFB), _p(alpha), _p(D), M, N, K, _p(ws),
                        0 if ws is None else ws.numel(), _stream(A.device)), "fp4_gemm")
    return D


def quantize_gemm(x, gs, B, SFB, alpha: torch.Tensor | None = None,
                  out: torch.Tensor | None = None) -> torch.Tensor:
    """D = gemm(quantize(x, "nvfp4", gs), B, SFB, alpha) in one call (one fused
    kernel for up to four rows)."""
    _need(x, torch.bfloat16, "x")
    _need(gs, torch.float32, "gs")
    _need(B, torch.uint8, "B")
    _need(SFB, torch.uint8, "SFB")
    M, K = x.shape
    N = B.shape[0]
    if alpha is not None:
        _need(alpha, torch.float32, "alpha")
    D = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _need(D, torch.bfloat16, "out")
    lib = load()
    ws = _workspace(lib.nvfp4_quantize_gemm_workspace_size(M, N, K), x.device)
    _check(lib.nvfp4_quantize_gemm(_p(x), _p(gs), _p(B), _p(SFB), _p(alpha), _p(D), M, N, K, _p(ws),
                                   0 if ws is None else ws.numel(), _stream(x.device)), "nvfp4_quantize_gemm")
    return D


def w4a16_gemm(A, B, SFB, alpha: torch.Tensor | None = None,
               out: torch.Tensor | None = None) -> torch.Tensor:
    """D = bf16(alpha * A @ dequant(B)^T); A bf16 [M, K], B [N, K/2] NVFP4."""
    _need(A, torch.bfloat16, "A")
    _need(B, torch.uint8, "B")
    _need(SFB, torch.uint8, "SFB")
    M, K = A.shape
    N = B.shape[0]
    if alpha is not None:
        _need(alpha, torch.float32, "alpha")
    D = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    _need(D, torch.bfloat16, "out")
    lib = load()
    ws = _workspace(lib.w4a16_gemm_workspace_size(M, N, K), A.device)
    _check(lib.w4a16_gemm(_p(A), _p(B), _p(SFB), _p(alpha), _p(D), M, N, K, _p(ws),
                          0 if ws is None else ws.numel(), _stream(A.device)), "w4a16_gemm")
    return D


SF_LAYOUTS = {"128x4": 0, "128x4_m8": 1}


def _sf_layout(layout) -> int:
    try:
        return SF_LAYOUTS[layout]
    except KeyError:
        raise ValueError(f"unknown scale layout {layout!r}") from None


def scales_swizzle(sf: torch.Tensor, layout="128x4", out: torch.Tensor | None = None) -> torch.Tensor:
    """Row-major [rows, kblocks] block scales -> padded swizzled [round_up(rows,128), round_up(kblocks,4)]."""
    _need(sf, torch.uint8, "sf")
    rows, kblocks = sf.shape
    R, C = -(-rows // 128) * 128, -(-kblocks // 4) * 4
    swz = out if out is not None else torch.empty((R, C), dtype=torch.uint8, device=sf.device)
    _need(swz, torch.uint8, "out")
    if swz.numel() != R * C:
        raise ValueError(f"out must hold {R * C} bytes")
    _check(load().fp4_scales_swizzle(_sf_layout(layout), _p(sf), rows, kblocks, _p(swz), _stream(sf.device)),
           "fp4_scales_swizzle")
    return swz


def scales_unswizzle(swz: torch.Tensor, rows: int, kblocks: int, layout="128x4",
                     out: torch.Tensor | None = None) -> torch.Tensor:
    """Padded swizzled block scales -> row-major [rows, kblocks] (the padding is dropped)."""
    _need(swz, torch.uint8, "swz")
    if swz.numel() != load().fp4_scales_swizzled_size(rows, kblocks):
        raise ValueError("swz does not hold the padded size of (rows, kblocks)")
    sf = out if out is not None else torch.empty((rows, kblocks), dtype=torch.uint8, device=swz.device)
    _need(sf, torch.uint8, "out")
    _check(load().fp4_scales_unswizzle(_sf_layout(layout), _p(swz), rows, kblocks, _p(sf), _stream(swz.device)),
           "fp4_scales_unswizzle")
    return sf


def moe_prep(topk_ids: torch.Tensor, num_experts: int):
    """(expert_offsets int32 [E+1], sorted_ids int32 [T*topk], sorted_tokens int32 [T*topk])."""
    _need(topk_ids, torch.int32, "topk_ids")
    T, topk = topk_ids.shape
    dev = topk_ids.device
    offsets = torch.empty(num_experts + 1, dtype=torch.int32, device=dev)
    sorted_ids = torch.empty(T * topk, dtype=torch.int32, device=dev)
    sorted_tokens = torch.empty(T * topk, dtype=torch.int32, device=dev)
    lib = load()
    ws = _workspace(lib.fp4_moe_prep_workspace_size(T, topk, num_experts), dev)
    _check(lib.fp4_moe_prep(_p(topk_ids), T, topk, num_experts, _p(offsets), _p(sorted_ids),
                            _p(sorted_tokens), _p(ws), 0 if ws is None else ws.numel(), _stream(dev)),
           "fp4_moe_prep")
    return offsets, sorted_ids, sorted_tokens


def mxfp4_moe_grouped_gemm(Aq, Asf, expert_offsets, W, Wsf, epilogue=MOE_STORE_BF16, *,
                           rows=None, a_row_index=None, out=None, out_q=None, out_sf=None,
                           sorted_ids=None, topk_weights=None, num_tokens=0, topk=0):
    """Grouped MXFP4 GEMM over expert-sorted rows; see the C header for epilogues.

    With a_row_index, problem row m reads row a_row_index[m] of Aq and `rows`
    defaults to len(a_row_index); otherwise rows = Aq.shape[0]."""
    for t, n in ((Aq, "Aq"), (Asf, "Asf"), (W, "W"), (Wsf, "Wsf")):
        _need(t, torch.uint8, n)
    _need(expert_offsets, torch.int32, "expert_offsets")
    a_total, K = Aq.shape[0], Aq.shape[1] * 2
    if a_row_index is not None:
        _need(a_row_index, torch.int32, "a_row_index")
        if rows is None:
            rows = a_row_index.numel()
    elif rows is None:
        rows = a_total
    E, N = W.shape[0], W.shape[1]
    dev = Aq.device
    if epilogue == MOE_STORE_BF16 and out is None:
        out = torch.empty((rows, N), dtype=torch.bfloat16, device=dev)
    if epilogue == MOE_SILU_MUL_QUANT:
        if out_q is None:
            out_q = torch.empty((rows, N // 4), dtype=torch.uint8, device=dev)
        if out_sf is None:
            out_sf = torch.empty((rows, N // 64), dtype=torch.uint8, device=dev)
    if epilogue == MOE_WEIGHTED_COMBINE:
        _need(sorted_ids, torch.int32, "sorted_ids")
        _need(topk_weights, torch.float32, "topk_weights")
        if out is None:
            out = torch.empty((num_tokens, N), dtype=torch.bfloat16, device=dev)
    args = MoeEpilogueArgs(
        out=None if out is None else out.data_ptr(),
        out_q=None if out_q is None else out_q.data_ptr(),
        out_sf=None if out_sf is None else out_sf.data_ptr(),
        sorted_ids=None if sorted_ids is None else sorted_ids.data_ptr(),
        topk_weights=None if topk_weights is None else topk_weights.data_ptr(),
        num_tokens=num_tokens, topk=topk)
    lib = load()
    ws = _workspace(lib.mxfp4_moe_grouped_gemm_workspace_size(rows, E, N, K, epilogue, num_tokens), dev)
    _check(lib.mxfp4_moe_grouped_gemm(_p(Aq), _p(Asf), a_total, _p(a_row_index), _p(expert_offsets), E,
                                      rows, _p(W), _p(Wsf), N, K, epilogue, ctypes.byref(args), _p(ws),
                                      0 if ws is None else ws.numel(), _stream(dev)),
           "mxfp4_moe_grouped_gemm")
    if epilogue == MOE_SILU_MUL_QUANT:
        return out_q, out_sf
    return out


def moe_layer(x, topk_ids, topk_weights, W13, W13sf, W2, W2sf):
    """The MXFP4 W4A4 MoE layer: routing prep -> MXFP4 quantisation of each
    token once -> gate_up grouped GEMM reading the activations by token, with
    the fused SiLU-gate + MXFP4 re-quant epilogue -> down grouped GEMM with the
    top-k weighted combine."""
    T, topk = topk_ids.shape
    E = W13.shape[0]
    offsets, sorted_ids, sorted_tokens = moe_prep(topk_ids, E)
    xq, xsf = quantize(x, "mxfp4")
    aq, asf = mxfp4_moe_grouped_gemm(xq, xsf, offsets, W13, W13sf, MOE_SILU_MUL_QUANT,
                                     a_row_index=sorted_tokens)
    return mxfp4_moe_grouped_gemm(aq, asf, offsets, W2, W2sf, MOE_WEIGHTED_COMBINE,
                                  sorted_ids=sorted_ids, topk_weights=topk_weights,
                                  num_tokens=T, topk=topk)


def nvfp4_experts_quantize(x, expert_offsets, gs_experts, row_map=None, q=None, sf=None):
    """NVFP4 rows grouped by expert: row r quantises x[row_map[r]] with the
    global scale gs_experts[e] of the expert that owns row r."""
    _need(x, torch.bfloat16, "x")
    _need(expert_offsets, torch.int32, "expert_offsets")
    _need(gs_experts, torch.float32, "gs_experts")
    R, K = x.shape
    rows_out = R
    if row_map is not None:
        _need(row_map, torch.int32, "row_map")
        rows_out = row_map.numel()
    E = expert_offsets.numel() - 1
    if q is None:
        q = torch.empty((rows_out, K // 2), dtype=torch.uint8, device=x.device)
    if sf is None:
        sf = torch.empty((rows_out, K // 16), dtype=torch.uint8, device=x.device)
    _check(load().nvfp4_experts_quantize(_p(x), R, K, _p(row_map), _p(expert_offsets), E, _p(gs_experts),
                                         rows_out, _p(q), _p(sf), _stream(x.device)), "nvfp4_experts_quantize")
    return q, sf


def nvfp4_moe_grouped_gemm(Aq, Asf, expert_offsets, W, Wsf, alpha_experts=None, epilogue=MOE_STORE_BF16, *,
                           out=None, out_q=None, out_sf=None, out_gs=None, sorted_ids=None,
                           topk_weights=None, num_tokens=0, topk=0):
    """Grouped NVFP4 GEMM over expert-sorted rows with per-expert alphas; see the C header."""
    for t, n in ((Aq, "Aq"), (Asf, "Asf"), (W, "W"), (Wsf, "Wsf")):
        _need(t, torch.uint8, n)
    _need(expert_offsets, torch.int32, "expert_offsets")
    if alpha_experts is not None:
        _need(alpha_experts, torch.float32, "alpha_experts")
    rows, K = Aq.shape[0], Aq.shape[1] * 2
    E, N = W.shape[0], W.shape[1]
    dev = Aq.device
    if epilogue == MOE_STORE_BF16 and out is None:
        out = torch.empty((rows, N), dtype=torch.bfloat16, device=dev)
    if epilogue == MOE_SILU_MUL_QUANT:
        _need(out_gs, torch.float32, "out_gs")
        if out_q is None:
            out_q = torch.empty((rows, N // 4), dtype=torch.uint8, device=dev)
        if out_sf is None:
            out_sf = torch.empty((rows, N // 32), dtype=torch.uint8, device=dev)
    if epilogue == MOE_WEIGHTED_COMBINE:
        _need(sorted_ids, torch.int32, "sorted_ids")
        _need(topk_weights, torch.float32, "topk_weights")
        if out is None:
            out = torch.empty((num_tokens, N), dtype=torch.bfloat16, device=dev)
    args = MoeEpilogueArgs(
        out=None if out is None else out.data_ptr(),
        out_q=None if out_q is None else out_q.data_ptr(),
        out_sf=None if out_sf is None else out_sf.data_ptr(),
        sorted_ids=None if sorted_ids is None else sorted_ids.data_ptr(),
        topk_weights=None if topk_weights is None else topk_weights.data_ptr(),
        num_tokens=num_tokens, topk=topk,
        out_gs=None if out_gs is None else out_gs.data_ptr())
    lib = load()
    ws = _workspace(lib.nvfp4_moe_grouped_gemm_workspace_size(rows, E, N, K, epilogue, num_tokens), dev)
    _check(lib.nvfp4_moe_grouped_gemm(_p(Aq), _p(Asf), _p(expert_offsets), E, rows, _p(W), _p(Wsf),
                                      _p(alpha_experts), N, K, epilogue, ctypes.byref(args), _p(ws),
                                      0 if ws is None else ws.numel(), _stream(dev)),
           "nvfp4_moe_grouped_gemm")
    if epilogue == MOE_SILU_MUL_QUANT:
        return out_q, out_sf
    return out


def nvfp4_moe_layer(x, topk_ids, topk_weights, W13, W13sf, W2, W2sf, gs1, alpha1, gs2, alpha2):
    """The NVFP4 W4A4 MoE layer: routing prep -> per-expert NVFP4 quantisation
    of each routed row (gs1[e]) -> gate_up grouped GEMM (alpha1[e]) with the
    fused SiLU-gate + NVFP4 re-quant epilogue (gs2[e]) -> down grouped GEMM
    (alpha2[e]) with the top-k weighted combine."""
    T, topk = topk_ids.shape
    E = W13.shape[0]
    offsets, sorted_ids, sorted_tokens = moe_prep(topk_ids, E)
    xq, xsf = nvfp4_experts_quantize(x, offsets, gs1, row_map=sorted_tokens)
    aq, asf = nvfp4_moe_grouped_gemm(xq, xsf, offsets, W13, W13sf, alpha1, MOE_SILU_MUL_QUANT, out_gs=gs2)
    return nvfp4_moe_grouped_gemm(aq, asf, offsets, W2, W2sf, alpha2, MOE_WEIGHTED_COMBINE,
                                  sorted_ids=sorted_ids, topk_weights=topk_weights,
                                  num_tokens=T, topk=topk)

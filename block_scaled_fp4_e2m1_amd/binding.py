"""Thin Python binding of libbsfp4 (ctypes).

Argument marshalling only: each function checks dtypes, contiguity and the
exact extents of every tensor it hands over (the C ABI sees raw pointers and
cannot check how large a buffer is, so an undersized scale or output tensor
must be refused here), then that all tensors sit on one GPU, allocates
outputs and workspace with torch (device memory and streams are all torch
is used for), and calls the library on the current HIP stream.  Shape errors
raise ValueError before anything reaches the library.  Every step of the
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
    "bsfp4_e2m1_convert": (ctypes.c_int, [ctypes.c_int, _c_ptr, _c_ptr, _c_i64, _c_ptr, _c_ptr]),
    "bsfp4_probe_mfma_flops": (_c_i64, [ctypes.c_int, ctypes.c_int]),
    "bsfp4_probe_mfma": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, _c_ptr]),
    "bsfp4_probe_read": (ctypes.c_int, [_c_ptr, _c_i64, _c_ptr]),
    "fp4_gemm_noalloc_max_workspace": (_c_size, []),
    "fp4_gemm_noalloc": (ctypes.c_int, [ctypes.c_int, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr,
                                        _c_i64, _c_i64, _c_i64, _c_ptr]),
}

CVT_F32 = 0
CVT_BF16_E8M0 = 1
CVT_F32_E8M0 = 2

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
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _dims(t, nd, name):
    if t.dim() != nd:
        raise ValueError(f"{name} must be {nd}-D, got shape {tuple(t.shape)}")


def _shape(t, shape, name):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _numel(t, n, name):
    if t.numel() != n:
        raise ValueError(f"{name} must hold {n} elements, got {t.numel()} (shape {tuple(t.shape)})")


def _device(*named):
    """Every given tensor must be a GPU tensor, all on the same device."""
    dev = None
    for t, name in named:
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be a device tensor (got {t.device})")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev}")
    return dev


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
    if x.numel() == 0:
        raise ValueError("x must not be empty")
    if out is not None:
        _need(out, torch.float32, "out")
        _numel(out, 1, "out")
    _device((x, "x"), (out, "out"))
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
    _dims(x, 2, "x")
    R, K = x.shape
    blk = 16 if f == NVFP4 else 32
    if K % blk:
        raise ValueError(f"K={K} is not a multiple of {blk}")
    if row_map is not None:
        _need(row_map, torch.int32, "row_map")
        _dims(row_map, 1, "row_map")
        rows_out = row_map.numel()
    else:
        rows_out = R
    if f == NVFP4:
        if gs is None:
            raise ValueError("NVFP4 quantisation needs the global scale gs")
        _need(gs, torch.float32, "gs")
        _numel(gs, 1, "gs")
    elif gs is not None:
        raise ValueError("MXFP4 quantisation takes no global scale")
    if q is not None:
        _need(q, torch.uint8, "q")
        _shape(q, (rows_out, K // 2), "q")
    if sf is not None:
        _need(sf, torch.uint8, "sf")
        _numel(sf, rows_out * (K // blk), "sf")
    _device((x, "x"), (row_map, "row_map"), (gs, "gs"), (q, "q"), (sf, "sf"))
    if q is None:
        q = torch.empty((rows_out, K // 2), dtype=torch.uint8, device=x.device)
    if sf is None:
        sf = torch.empty((rows_out, K // blk), dtype=torch.uint8, device=x.device)
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
    _dims(A, 2, "A")
    _dims(B, 2, "B")
    M, K = A.shape[0], A.shape[1] * 2
    N = B.shape[0]
    if B.shape[1] * 2 != K:
        raise ValueError(f"A has K={K} but B has K={B.shape[1] * 2}")
    blk = 16 if f == NVFP4 else 32
    if K % blk:
        raise ValueError(f"K={K} is not a multiple of {blk}")
    _numel(SFA, M * (K // blk), "SFA")
    _numel(SFB, N * (K // blk), "SFB")
    if alpha is not None:
        _need(alpha, torch.float32, "alpha")
        _numel(alpha, 1, "alpha")
    if out is not None:
        _need(out, torch.bfloat16, "out")
        _shape(out, (M, N), "out")
    _device((A, "A"), (SFA, "SFA"), (B, "B"), (SFB, "SFB"), (alpha, "alpha"), (out, "out"))
    D = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
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
    _dims(x, 2, "x")
    _dims(B, 2, "B")
    M, K = x.shape
    N = B.shape[0]
    if B.shape[1] * 2 != K:
        raise ValueError(f"x has K={K} but B has K={B.shape[1] * 2}")
    if K % 16:
        raise ValueError(f"K={K} is not a multiple of 16")
    _numel(gs, 1, "gs")
    _numel(SFB, N * (K // 16), "SFB")
    if alpha is not None:
        _need(alpha, torch.float32, "alpha")
        _numel(alpha, 1, "alpha")
    if out is not None:
        _need(out, torch.bfloat16, "out")
        _shape(out, (M, N), "out")
    _device((x, "x"), (gs, "gs"), (B, "B"), (SFB, "SFB"), (alpha, "alpha"), (out, "out"))
    D = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
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
    _dims(A, 2, "A")
    _dims(B, 2, "B")
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] * 2 != K:
        raise ValueError(f"A has K={K} but B has K={B.shape[1] * 2}")
    if K % 16:
        raise ValueError(f"K={K} is not a multiple of 16")
    _numel(SFB, N * (K // 16), "SFB")
    if alpha is not None:
        _need(alpha, torch.float32, "alpha")
        _numel(alpha, 1, "alpha")
    if out is not None:
        _need(out, torch.bfloat16, "out")
        _shape(out, (M, N), "out")
    _device((A, "A"), (B, "B"), (SFB, "SFB"), (alpha, "alpha"), (out, "out"))
    D = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    lib = load()
    ws = _workspace(lib.w4a16_gemm_workspace_size(M, N, K), A.device)
    _check(lib.w4a16_gemm(_p(A), _p(B), _p(SFB), _p(alpha), _p(D), M, N, K, _p(ws),
                          0 if ws is None else ws.numel(), _stream(A.device)), "w4a16_gemm")
    return D


def e2m1_convert(values: torch.Tensor, scale_codes: torch.Tensor | None = None) -> torch.Tensor:
    """E2M1 codes of value pairs by the kernels' own converters (diagnostic).

    values: float32 [2n] (scale 1 without scale_codes, else pair i divided by
    2^(scale_codes[i] - 127)) or bf16 [2n] (scale_codes required); n % 4 == 0.
    Returns uint8 [n]: code of value 2i in the low nibble of byte i."""
    if not isinstance(values, torch.Tensor) or values.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("values must be a float32 or bfloat16 tensor")
    _need(values, values.dtype, "values")
    _dims(values, 1, "values")
    if values.numel() % 8:
        raise ValueError("values must hold a multiple of 8 elements (4 pairs)")
    pairs = values.numel() // 2
    if values.dtype == torch.bfloat16:
        if scale_codes is None:
            raise ValueError("bf16 values need scale_codes")
        mode = CVT_BF16_E8M0
    else:
        mode = CVT_F32 if scale_codes is None else CVT_F32_E8M0
    if scale_codes is not None:
        _need(scale_codes, torch.uint8, "scale_codes")
        _numel(scale_codes, pairs, "scale_codes")
    dev = _device((values, "values"), (scale_codes, "scale_codes"))
    codes = torch.empty(pairs, dtype=torch.uint8, device=dev)
    _check(load().bsfp4_e2m1_convert(mode, _p(values), _p(scale_codes), pairs, _p(codes), _stream(dev)),
           "bsfp4_e2m1_convert")
    return codes


SF_LAYOUTS = {"128x4": 0, "128x4_m8": 1}


def _sf_layout(layout) -> int:
    try:
        return SF_LAYOUTS[layout]
    except KeyError:
        raise ValueError(f"unknown scale layout {layout!r}") from None


def scales_swizzle(sf: torch.Tensor, layout="128x4", out: torch.Tensor | None = None) -> torch.Tensor:
    """Row-major [rows, kblocks] block scales -> padded swizzled [round_up(rows,128), round_up(kblocks,4)]."""
    _need(sf, torch.uint8, "sf")
    _dims(sf, 2, "sf")
    rows, kblocks = sf.shape
    R, C = -(-rows // 128) * 128, -(-kblocks // 4) * 4
    if out is not None:
        _need(out, torch.uint8, "out")
        _numel(out, R * C, "out")
    _device((sf, "sf"), (out, "out"))
    swz = out if out is not None else torch.empty((R, C), dtype=torch.uint8, device=sf.device)
    _check(load().fp4_scales_swizzle(_sf_layout(layout), _p(sf), rows, kblocks, _p(swz), _stream(sf.device)),
           "fp4_scales_swizzle")
    return swz


def scales_unswizzle(swz: torch.Tensor, rows: int, kblocks: int, layout="128x4",
                     out: torch.Tensor | None = None) -> torch.Tensor:
    """Padded swizzled block scales -> row-major [rows, kblocks] (the padding is dropped)."""
    _need(swz, torch.uint8, "swz")
    if rows < 0 or kblocks <= 0:
        raise ValueError(f"need rows >= 0 and kblocks > 0 (rows={rows}, kblocks={kblocks})")
    _numel(swz, (-(-rows // 128) * 128) * (-(-kblocks // 4) * 4), "swz")
    if out is not None:
        _need(out, torch.uint8, "out")
        _numel(out, rows * kblocks, "out")
    _device((swz, "swz"), (out, "out"))
    sf = out if out is not None else torch.empty((rows, kblocks), dtype=torch.uint8, device=swz.device)
    _check(load().fp4_scales_unswizzle(_sf_layout(layout), _p(swz), rows, kblocks, _p(sf), _stream(swz.device)),
           "fp4_scales_unswizzle")
    return sf


def moe_prep(topk_ids: torch.Tensor, num_experts: int):
    """(expert_offsets int32 [E+1], sorted_ids int32 [T*topk], sorted_tokens int32 [T*topk])."""
    _need(topk_ids, torch.int32, "topk_ids")
    _dims(topk_ids, 2, "topk_ids")
    if num_experts <= 0:
        raise ValueError(f"num_experts must be > 0, got {num_experts}")
    T, topk = topk_ids.shape
    dev = _device((topk_ids, "topk_ids"))
    offsets = torch.empty(num_experts + 1, dtype=torch.int32, device=dev)
    sorted_ids = torch.empty(T * topk, dtype=torch.int32, device=dev)
    sorted_tokens = torch.empty(T * topk, dtype=torch.int32, device=dev)
    lib = load()
    ws = _workspace(lib.fp4_moe_prep_workspace_size(T, topk, num_experts), dev)
    _check(lib.fp4_moe_prep(_p(topk_ids), T, topk, num_experts, _p(offsets), _p(sorted_ids),
                            _p(sorted_tokens), _p(ws), 0 if ws is None else ws.numel(), _stream(dev)),
           "fp4_moe_prep")
    return offsets, sorted_ids, sorted_tokens


def _moe_common(K, blk, E, N, W, Asf, a_rows, Wsf, expert_offsets):
    """Extents shared by the grouped GEMMs: W [E, N, K/2] codes, its scales,
    the activation scales and the expert offsets."""
    if K % blk:
        raise ValueError(f"K={K} is not a multiple of {blk}")
    if W.shape[2] * 2 != K:
        raise ValueError(f"Aq has K={K} but W has K={W.shape[2] * 2}")
    _numel(Asf, a_rows * (K // blk), "Asf")
    _numel(Wsf, E * N * (K // blk), "Wsf")
    _numel(expert_offsets, E + 1, "expert_offsets")


def _moe_outputs(epilogue, rows, N, act_blk, out, out_q, out_sf, sorted_ids, topk_weights, num_tokens, topk):
    """Output extents of each epilogue (act_blk: 64 values of N per MXFP4
    act scale byte, i.e. 32 act values; 32 of N per NVFP4 act scale byte)."""
    if epilogue == MOE_STORE_BF16:
        if out is not None:
            _need(out, torch.bfloat16, "out")
            _shape(out, (rows, N), "out")
    elif epilogue == MOE_SILU_MUL_QUANT:
        if N % 64:
            raise ValueError(f"SILU_MUL_QUANT needs N % 64 == 0 (got N={N})")
        if out_q is not None:
            _need(out_q, torch.uint8, "out_q")
            _shape(out_q, (rows, N // 4), "out_q")
        if out_sf is not None:
            _need(out_sf, torch.uint8, "out_sf")
            _numel(out_sf, rows * (N // act_blk), "out_sf")
    elif epilogue == MOE_WEIGHTED_COMBINE:
        if sorted_ids is None or topk_weights is None:
            raise ValueError("WEIGHTED_COMBINE needs sorted_ids and topk_weights")
        if num_tokens <= 0 or topk <= 0 or num_tokens * topk != rows:
            raise ValueError(f"WEIGHTED_COMBINE needs num_tokens * topk == rows "
                             f"(num_tokens={num_tokens}, topk={topk}, rows={rows})")
        _need(sorted_ids, torch.int32, "sorted_ids")
        _numel(sorted_ids, rows, "sorted_ids")
        _need(topk_weights, torch.float32, "topk_weights")
        _numel(topk_weights, rows, "topk_weights")
        if out is not None:
            _need(out, torch.bfloat16, "out")
            _shape(out, (num_tokens, N), "out")
    else:
        raise ValueError(f"unknown epilogue {epilogue!r}")


def _moe_layer_shapes(x, topk_ids, topk_weights, W13, W2):
    _need(x, torch.bfloat16, "x")
    _need(topk_ids, torch.int32, "topk_ids")
    _need(topk_weights, torch.float32, "topk_weights")
    _dims(x, 2, "x")
    _dims(topk_ids, 2, "topk_ids")
    _dims(W13, 3, "W13")
    _dims(W2, 3, "W2")
    T, H = x.shape
    _shape(topk_weights, topk_ids.shape, "topk_weights")
    if topk_ids.shape[0] != T:
        raise ValueError(f"x has {T} tokens but topk_ids has {topk_ids.shape[0]}")
    E, two_i, h2 = W13.shape
    if h2 * 2 != H:
        raise ValueError(f"W13 has K={h2 * 2} but x has hidden size {H}")
    if two_i % 2:
        raise ValueError("W13 must hold gate and up rows (an even row count)")
    if tuple(W2.shape) != (E, H, two_i // 4):
        raise ValueError(f"W2 must have shape {(E, H, two_i // 4)}, got {tuple(W2.shape)}")


def mxfp4_moe_grouped_gemm(Aq, Asf, expert_offsets, W, Wsf, epilogue=MOE_STORE_BF16, *,
                           rows=None, a_row_index=None, out=None, out_q=None, out_sf=None,
                           sorted_ids=None, topk_weights=None, num_tokens=0, topk=0):
    """Grouped MXFP4 GEMM over expert-sorted rows; see the C header for epilogues.

    With a_row_index, problem row m reads row a_row_index[m] of Aq and `rows`
    defaults to len(a_row_index); otherwise rows = Aq.shape[0]."""
    for t, n in ((Aq, "Aq"), (Asf, "Asf"), (W, "W"), (Wsf, "Wsf")):
        _need(t, torch.uint8, n)
    _need(expert_offsets, torch.int32, "expert_offsets")
    _dims(Aq, 2, "Aq")
    _dims(W, 3, "W")
    a_total, K = Aq.shape[0], Aq.shape[1] * 2
    if a_row_index is not None:
        _need(a_row_index, torch.int32, "a_row_index")
        _dims(a_row_index, 1, "a_row_index")
        if rows is None:
            rows = a_row_index.numel()
        elif rows > a_row_index.numel():
            raise ValueError(f"rows={rows} exceeds len(a_row_index)={a_row_index.numel()}")
    elif rows is None:
        rows = a_total
    elif rows != a_total:
        raise ValueError(f"without a_row_index rows ({rows}) must equal Aq.shape[0] ({a_total})")
    E, N = W.shape[0], W.shape[1]
    _moe_common(K, 32, E, N, W, Asf, a_total, Wsf, expert_offsets)
    _moe_outputs(epilogue, rows, N, 64, out, out_q, out_sf, sorted_ids, topk_weights, num_tokens, topk)
    dev = _device((Aq, "Aq"), (Asf, "Asf"), (W, "W"), (Wsf, "Wsf"), (expert_offsets, "expert_offsets"),
                  (a_row_index, "a_row_index"), (out, "out"), (out_q, "out_q"), (out_sf, "out_sf"),
                  (sorted_ids, "sorted_ids"), (topk_weights, "topk_weights"))
    if epilogue == MOE_STORE_BF16 and out is None:
        out = torch.empty((rows, N), dtype=torch.bfloat16, device=dev)
    if epilogue == MOE_SILU_MUL_QUANT:
        if out_q is None:
            out_q = torch.empty((rows, N // 4), dtype=torch.uint8, device=dev)
        if out_sf is None:
            out_sf = torch.empty((rows, N // 64), dtype=torch.uint8, device=dev)
    if epilogue == MOE_WEIGHTED_COMBINE and out is None:
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
    _moe_layer_shapes(x, topk_ids, topk_weights, W13, W2)
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
    _dims(x, 2, "x")
    R, K = x.shape
    if K % 16:
        raise ValueError(f"K={K} is not a multiple of 16")
    rows_out = R
    if row_map is not None:
        _need(row_map, torch.int32, "row_map")
        _dims(row_map, 1, "row_map")
        rows_out = row_map.numel()
    E = expert_offsets.numel() - 1
    if E <= 0:
        raise ValueError("expert_offsets must hold E + 1 >= 2 entries")
    _numel(gs_experts, E, "gs_experts")
    if q is not None:
        _need(q, torch.uint8, "q")
        _shape(q, (rows_out, K // 2), "q")
    if sf is not None:
        _need(sf, torch.uint8, "sf")
        _numel(sf, rows_out * (K // 16), "sf")
    _device((x, "x"), (expert_offsets, "expert_offsets"), (gs_experts, "gs_experts"), (row_map, "row_map"),
            (q, "q"), (sf, "sf"))
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
    _dims(Aq, 2, "Aq")
    _dims(W, 3, "W")
    rows, K = Aq.shape[0], Aq.shape[1] * 2
    E, N = W.shape[0], W.shape[1]
    _moe_common(K, 16, E, N, W, Asf, rows, Wsf, expert_offsets)
    if alpha_experts is not None:
        _need(alpha_experts, torch.float32, "alpha_experts")
        _numel(alpha_experts, E, "alpha_experts")
    if epilogue == MOE_SILU_MUL_QUANT:
        if out_gs is None:
            raise ValueError("SILU_MUL_QUANT needs out_gs (one global scale per expert)")
        _need(out_gs, torch.float32, "out_gs")
        _numel(out_gs, E, "out_gs")
    _moe_outputs(epilogue, rows, N, 32, out, out_q, out_sf, sorted_ids, topk_weights, num_tokens, topk)
    dev = _device((Aq, "Aq"), (Asf, "Asf"), (W, "W"), (Wsf, "Wsf"), (expert_offsets, "expert_offsets"),
                  (alpha_experts, "alpha_experts"), (out, "out"), (out_q, "out_q"), (out_sf, "out_sf"),
                  (out_gs, "out_gs"), (sorted_ids, "sorted_ids"), (topk_weights, "topk_weights"))
    if epilogue == MOE_STORE_BF16 and out is None:
        out = torch.empty((rows, N), dtype=torch.bfloat16, device=dev)
    if epilogue == MOE_SILU_MUL_QUANT:
        if out_q is None:
            out_q = torch.empty((rows, N // 4), dtype=torch.uint8, device=dev)
        if out_sf is None:
            out_sf = torch.empty((rows, N // 32), dtype=torch.uint8, device=dev)
    if epilogue == MOE_WEIGHTED_COMBINE and out is None:
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
    _moe_layer_shapes(x, topk_ids, topk_weights, W13, W2)
    T, topk = topk_ids.shape
    E = W13.shape[0]
    offsets, sorted_ids, sorted_tokens = moe_prep(topk_ids, E)
    xq, xsf = nvfp4_experts_quantize(x, offsets, gs1, row_map=sorted_tokens)
    aq, asf = nvfp4_moe_grouped_gemm(xq, xsf, offsets, W13, W13sf, alpha1, MOE_SILU_MUL_QUANT, out_gs=gs2)
    return nvfp4_moe_grouped_gemm(aq, asf, offsets, W2, W2sf, alpha2, MOE_WEIGHTED_COMBINE,
                                  sorted_ids=sorted_ids, topk_weights=topk_weights,
                                  num_tokens=T, topk=topk)

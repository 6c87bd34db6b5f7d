"""CPU checks of the C ABI: the library loads, exports every function that
include/bsfp4.h declares, and rejects invalid arguments before touching a
device (no kernel is ever launched here)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsfp4.h")
LIB = os.path.join(ROOT, "block_scaled_fp4_e2m1_amd", "lib", "libbsfp4.so")

OK, INVALID, SHAPE, ALIGN, WORKSPACE = 0, 1, 2, 3, 4


def declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"BSFP4_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libbsfp4.so is not built (run __graft_entry__.build())")
    from block_scaled_fp4_e2m1_amd import binding
    return binding.load()


def test_header_declares_the_hot_path():
    names = declared()
    for fn in ["fp4_quantize", "fp4_gemm", "w4a16_gemm", "mxfp4_moe_grouped_gemm", "fp4_moe_prep",
               "fp4_global_scale", "bsfp4_last_error", "nvfp4_experts_quantize", "nvfp4_moe_grouped_gemm",
               "nvfp4_quantize_gemm"]:
        assert fn in names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\sT\s(\w+)$", out, re.M))
    missing = [n for n in declared() if n not in exported]
    assert not missing, f"declared but not exported: {missing}"
    # nothing else leaks out of the library
    extra = [n for n in exported if not (n.startswith("fp4_") or n.startswith("bsfp4_")
                                         or n.startswith("w4a16_") or n.startswith("mxfp4_")
                                         or n.startswith("nvfp4_"))]
    assert not extra, extra


def test_status_strings(lib):
    assert lib.bsfp4_version() >= 100
    assert lib.bsfp4_status_string(SHAPE) == b"unsupported shape"
    assert lib.bsfp4_status_string(99) == b"unknown status"


FAKE = 0x100000  # never dereferenced: every call below fails validation first


def _err(lib):
    return lib.bsfp4_last_error().decode()


def test_quantize_validation(lib):
    f = lib.fp4_quantize
    assert f(7, FAKE, 4, 64, FAKE, None, 4, FAKE, FAKE, None) == INVALID
    assert f(0, FAKE, 4, 24, FAKE, None, 4, FAKE, FAKE, None) == SHAPE and "multiple of 16" in _err(lib)
    assert f(1, FAKE, 4, 48, None, None, 4, FAKE, FAKE, None) == SHAPE and "multiple of 32" in _err(lib)
    assert f(0, FAKE, 4, 64, None, None, 4, FAKE, FAKE, None) == INVALID and "gs" in _err(lib)
    assert f(1, FAKE, 4, 64, FAKE, None, 4, FAKE, FAKE, None) == INVALID
    assert f(0, FAKE + 8, 4, 64, FAKE, None, 4, FAKE, FAKE, None) == ALIGN
    assert f(0, FAKE, 4, 64, FAKE + 2, None, 4, FAKE, FAKE, None) == ALIGN
    assert f(0, FAKE, 4, 64, FAKE, None, 5, FAKE, FAKE, None) == SHAPE  # rows_out != rows_in
    assert f(0, FAKE, -1, 64, FAKE, None, 4, FAKE, FAKE, None) == SHAPE
    assert f(0, FAKE, 4, 64, FAKE, None, 0, FAKE, FAKE, None) == SHAPE  # rows_out != rows_in
    assert f(0, None, 0, 64, FAKE, None, 0, None, None, None) == OK     # empty: a no-op
    assert f(0, FAKE, 4, 64, FAKE, None, 4, None, FAKE, None) == INVALID


def test_gemm_validation(lib):
    f = lib.fp4_gemm
    args = lambda **kw: [kw.get("fmt", 0), kw.get("A", FAKE), kw.get("SFA", FAKE), kw.get("B", FAKE),
                         kw.get("SFB", FAKE), kw.get("alpha", FAKE), kw.get("D", FAKE),
                         kw.get("M", 64), kw.get("N", 64), kw.get("K", 64), kw.get("ws", None),
                         kw.get("ws_bytes", 0), None]
    assert f(*args(fmt=3)) == INVALID
    assert f(*args(N=48)) == SHAPE and "N=48" in _err(lib)
    assert f(*args(K=80)) == SHAPE
    assert f(*args(M=-1)) == SHAPE
    assert f(*args(A=None)) == INVALID
    assert f(*args(B=FAKE + 4)) == ALIGN
    assert f(*args(alpha=FAKE + 2)) == ALIGN
    assert f(*args(M=0, A=None, SFA=None, D=None)) == OK  # empty output: nothing to do
    # MXFP4 operands address with 32-bit offsets: 2^31 bytes or more are refused
    # before any device query or launch
    assert f(*args(fmt=1, M=1 << 16, K=1 << 16)) == SHAPE and "2^31" in _err(lib)
    assert f(*args(fmt=1, N=1 << 16, K=1 << 16)) == SHAPE and "2^31" in _err(lib)


def test_mxfp4_grouped_validation(lib):
    from block_scaled_fp4_e2m1_amd.binding import MoeEpilogueArgs
    g = lib.mxfp4_moe_grouped_gemm
    ep = MoeEpilogueArgs(out=FAKE)

    def call(a_total=64, rows=64, N=128, K=64, E=4, epi=0, idx=None):
        return g(FAKE, FAKE, a_total, idx, FAKE, E, rows, FAKE, FAKE, N, K, epi, ctypes.byref(ep), None, 0, None)

    assert call(epi=7) == INVALID
    assert call(K=48) == SHAPE
    assert call(N=96, epi=1) == SHAPE and "N % 64" in _err(lib)
    assert call(a_total=32) == SHAPE               # without an index, a_rows_total must equal rows
    # 32-bit offsets: Aq and one expert's W must stay below 2^31 bytes
    assert call(a_total=1 << 16, rows=1 << 16, K=1 << 16) == SHAPE and "2^31" in _err(lib)
    assert call(a_total=64, rows=64, N=1 << 16, K=1 << 16) == SHAPE and "2^31" in _err(lib)
    assert call(a_total=1 << 16, rows=64, K=1 << 16, idx=FAKE) == SHAPE and "2^31" in _err(lib)


def test_gemm_noalloc_validation(lib):
    f = lib.fp4_gemm_noalloc
    assert lib.fp4_gemm_noalloc_max_workspace() == 32 << 20
    args = lambda **kw: [kw.get("fmt", 0), kw.get("A", FAKE), kw.get("SFA", FAKE), kw.get("B", FAKE),
                         kw.get("SFB", FAKE), kw.get("alpha", FAKE), kw.get("D", FAKE),
                         kw.get("M", 64), kw.get("N", 64), kw.get("K", 64), None]
    assert f(*args(fmt=3)) == INVALID
    assert f(*args(N=48)) == SHAPE
    assert f(*args(A=None)) == INVALID
    assert f(*args(D=FAKE + 8)) == ALIGN
    assert f(*args(fmt=1, M=1 << 16, K=1 << 16)) == SHAPE
    # partials beyond the static scratch: refused before any device query
    assert lib.fp4_gemm_workspace_size(0, 1024, 4096, 7168) > (32 << 20)
    assert f(*args(M=1024, N=4096, K=7168)) == WORKSPACE and "static scratch" in _err(lib)
    assert f(*args(M=0, A=None, SFA=None, D=None)) == OK


def test_e2m1_convert_validation(lib):
    f = lib.bsfp4_e2m1_convert
    assert f(3, FAKE, None, 8, FAKE, None) == INVALID
    assert f(0, FAKE, None, 6, FAKE, None) == SHAPE          # pairs % 4
    assert f(0, FAKE, None, -4, FAKE, None) == SHAPE
    assert f(0, FAKE, FAKE, 8, FAKE, None) == INVALID        # the unit-scale form takes no scales
    assert f(1, FAKE, None, 8, FAKE, None) == INVALID        # the E8M0 forms need them
    assert f(2, FAKE + 4, FAKE, 8, FAKE, None) == ALIGN
    assert f(0, None, None, 0, None, None) == OK             # empty: a no-op


def test_global_scale_validation(lib):
    f = lib.fp4_global_scale
    assert f(FAKE, 0, FAKE, FAKE, 1024, None) == SHAPE
    need = lib.fp4_global_scale_workspace_size(1 << 20)
    assert need > 0
    assert f(FAKE, 1 << 20, FAKE, FAKE, need - 4, None) == WORKSPACE
    assert f(FAKE + 1, 1 << 20, FAKE, FAKE, need, None) == ALIGN


def test_scale_layout_validation(lib):
    assert lib.fp4_scales_swizzled_size(200, 13) == 256 * 16
    assert lib.fp4_scales_swizzled_size(0, 13) == 0
    f, g = lib.fp4_scales_swizzle, lib.fp4_scales_unswizzle
    assert f(2, FAKE, 4, 8, FAKE, None) == INVALID and "layout" in _err(lib)
    assert f(0, FAKE, 4, 0, FAKE, None) == SHAPE
    assert f(1, FAKE, -1, 8, FAKE, None) == SHAPE
    assert f(0, None, 4, 8, FAKE, None) == INVALID
    assert f(0, FAKE, 4, 8, FAKE + 2, None) == ALIGN
    assert g(0, FAKE + 2, 4, 8, FAKE, None) == ALIGN
    assert g(1, FAKE, 4, 8, None, None) == INVALID
    assert f(0, FAKE, 1 << 20, 1 << 12, FAKE, None) == SHAPE and "2^31" in _err(lib)
    assert f(0, None, 0, 8, None, None) == OK  # empty: a no-op


def test_nvfp4_moe_validation(lib):
    import ctypes

    from block_scaled_fp4_e2m1_amd.binding import MoeEpilogueArgs
    q = lib.nvfp4_experts_quantize
    #        x     rows K   row_map offs  E  gs    rows_out q     sf
    assert q(FAKE, 8, 40, None, FAKE, 4, FAKE, 8, FAKE, FAKE, None) == SHAPE and "multiple of 16" in _err(lib)
    assert q(FAKE, 8, 64, None, FAKE, 0, FAKE, 8, FAKE, FAKE, None) == SHAPE
    assert q(FAKE, 8, 64, None, FAKE, 1025, FAKE, 8, FAKE, FAKE, None) == SHAPE
    assert q(FAKE, 8, 64, None, FAKE, 4, FAKE, 9, FAKE, FAKE, None) == SHAPE  # rows_out != rows_in
    assert q(FAKE, 8, 64, None, None, 4, FAKE, 8, FAKE, FAKE, None) == INVALID
    assert q(FAKE, 8, 64, None, FAKE, 4, None, 8, FAKE, FAKE, None) == INVALID
    assert q(FAKE, 8, 64, None, FAKE, 4, FAKE + 2, 8, FAKE, FAKE, None) == ALIGN
    assert q(FAKE, 8, 64, FAKE + 1, FAKE, 4, FAKE, 8, FAKE, FAKE, None) == ALIGN
    assert q(None, 0, 64, None, FAKE, 4, FAKE, 0, None, None, None) == OK  # empty: a no-op

    g = lib.nvfp4_moe_grouped_gemm
    ep = MoeEpilogueArgs(out=FAKE, out_q=FAKE, out_sf=FAKE, out_gs=FAKE)

    def call(epi=0, E=4, rows=64, N=128, K=64, alpha=FAKE, args=ep, ws=None, ws_bytes=0, Aq=FAKE):
        return g(Aq, FAKE, FAKE, E, rows, FAKE, FAKE, alpha, N, K, epi, ctypes.byref(args) if args else None,
                 ws, ws_bytes, None)

    assert call(epi=3) == INVALID
    assert call(args=None) == INVALID
    assert call(E=0) == SHAPE and call(E=1025) == SHAPE
    assert call(K=48) == SHAPE and call(N=48) == SHAPE
    assert call(epi=1, N=96) == SHAPE and "N % 64" in _err(lib)
    assert call(N=1 << 16, K=1 << 16) == SHAPE and "2^31" in _err(lib)
    assert call(alpha=FAKE + 2) == ALIGN
    assert call(Aq=None) == INVALID
    assert call(epi=1, args=MoeEpilogueArgs(out_q=FAKE, out_sf=FAKE)) == INVALID and "out_gs" in _err(lib)
    assert call(epi=1, args=MoeEpilogueArgs(out_q=FAKE, out_sf=FAKE + 1, out_gs=FAKE)) == ALIGN
    comb = MoeEpilogueArgs(out=FAKE, sorted_ids=FAKE, topk_weights=FAKE, num_tokens=8, topk=8)
    assert call(epi=2, args=comb) == WORKSPACE
    assert call(epi=2, args=MoeEpilogueArgs(out=FAKE, sorted_ids=FAKE, topk_weights=FAKE, num_tokens=8,
                                            topk=4)) == SHAPE
    assert lib.nvfp4_moe_grouped_gemm_workspace_size(64, 4, 128, 64, 2, 8) == 64 * 128 * 4
    assert lib.nvfp4_moe_grouped_gemm_workspace_size(64, 4, 128, 64, 1, 8) == 0
    assert call(rows=0, Aq=None) == OK  # no rows: nothing to do


def test_quantize_gemm_validation(lib):
    f = lib.nvfp4_quantize_gemm
    args = lambda **kw: [kw.get("x", FAKE), kw.get("gs", FAKE), kw.get("B", FAKE), kw.get("SFB", FAKE),
                         kw.get("alpha", None), kw.get("D", FAKE), kw.get("M", 300), kw.get("N", 64),
                         kw.get("K", 64), kw.get("ws", None), kw.get("ws_bytes", 0), None]
    assert f(*args(K=48)) == SHAPE and f(*args(N=48)) == SHAPE and f(*args(M=-1)) == SHAPE
    assert f(*args(gs=None)) == INVALID and "gs" in _err(lib)
    assert f(*args(gs=FAKE + 2)) == ALIGN
    assert f(*args(x=None)) == INVALID
    assert f(*args(alpha=FAKE + 1)) == ALIGN
    need = lib.nvfp4_quantize_gemm_workspace_size(300, 64, 64)
    assert need >= 300 * 32 + 300 * 4
    assert f(*args()) == WORKSPACE
    assert f(*args(ws=FAKE + 8, ws_bytes=need)) == ALIGN
    assert f(*args(M=0, x=None, D=None)) == OK
    assert lib.nvfp4_quantize_gemm_workspace_size(0, 64, 64) == 0


def test_probe_validation(lib):
    flops = lib.bsfp4_probe_mfma_flops
    # flops per launch scale with iters; the 64-deep fp8 / fp4 forms do 4x the fp16 work per MFMA
    assert flops(0, 8) > 0 and flops(0, 16) == 2 * flops(0, 8)
    assert flops(3, 8) == 4 * flops(0, 8) and flops(6, 8) == flops(3, 8)
    assert flops(7, 8) == flops(0, 8) and flops(2, 8) == flops(3, 8)
    for kind, iters in ((-1, 8), (8, 8), (0, 0), (0, (1 << 24) + 1), (6, 6), (7, 2)):
        assert flops(kind, iters) == 0, (kind, iters)
    probe = lib.bsfp4_probe_mfma
    assert probe(8, 16, None) == INVALID
    assert probe(-1, 16, None) == INVALID
    assert probe(0, 0, None) == SHAPE
    assert probe(6, 6, None) == SHAPE and "multiple of 4" in _err(lib)
    assert probe(7, 1 << 25, None) == SHAPE
    read = lib.bsfp4_probe_read
    assert read(FAKE, 0, None) == SHAPE
    assert read(FAKE, 24, None) == SHAPE
    assert read(None, 32, None) == INVALID

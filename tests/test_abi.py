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
               "fp4_global_scale", "bsfp4_last_error"]:
        assert fn in names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\sT\s(\w+)$", out, re.M))
    missing = [n for n in declared() if n not in exported]
    assert not missing, f"declared but not exported: {missing}"
    # nothing else leaks out of the library
    extra = [n for n in exported if not (n.startswith("fp4_") or n.startswith("bsfp4_")
                                         or n.startswith("w4a16_") or n.startswith("mxfp4_"))]
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

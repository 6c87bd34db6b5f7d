"""fp4_gemm_noalloc (the allocation-free GEMM entry point) against fp4_gemm.

Called through the C ABI with ctypes.  Two calls in a row, the second with a
smaller problem, both of shapes whose K split keeps FP32 partials in the
library's static scratch; each output must equal fp4_gemm's bit for bit (same
kernels, same plan) and meet the oracle's tolerance rule.  A shape needing more
partials than the scratch holds is refused before any launch.
"""
import ctypes

import numpy as np
import pytest
import torch

import block_scaled_fp4_e2m1_amd as bs
from block_scaled_fp4_e2m1_amd import binding as B
from oracle import gemm as OG
from oracle import tolerance as TOL
from gpu_helpers import DEV, dev_f32, dev_u8, host_bf16_bits, mxfp4_problem, nvfp4_problem

pytestmark = pytest.mark.gpu

WORKSPACE = 4


def _noalloc(lib, fmt, aq, sfa, bq, sfb, alpha, out, M, N, K):
    return lib.fp4_gemm_noalloc(fmt, B._p(aq), B._p(sfa), B._p(bq), B._p(sfb), B._p(alpha), B._p(out),
                                M, N, K, B._stream(torch.device(DEV)))


def test_noalloc_matches_fp4_gemm_on_two_calls():
    lib = bs.load()
    assert lib.fp4_gemm_noalloc_max_workspace() == 32 << 20
    for M, N, K, seed in [(128, 4096, 7168, 300), (32, 2048, 4096, 310)]:
        need = lib.fp4_gemm_workspace_size(0, M, N, K)
        assert 0 < need <= lib.fp4_gemm_noalloc_max_workspace(), (M, N, K, need)
        aq, sfa, bq, sfb, alpha = nvfp4_problem(M, N, K, seed)
        daq, dsfa, dbq, dsfb, dal = dev_u8(aq), dev_u8(sfa), dev_u8(bq), dev_u8(sfb), dev_f32([alpha])
        ref = bs.gemm(daq, dsfa, dbq, dsfb, dal)
        out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
        st = _noalloc(lib, 0, daq, dsfa, dbq, dsfb, dal, out, M, N, K)
        assert st == 0, lib.bsfp4_last_error().decode()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"noalloc differs from fp4_gemm at {M}x{N}x{K}"
        rows = np.unique(np.linspace(0, M - 1, 16).astype(int))
        want = OG.nvfp4_gemm(aq[rows], sfa[rows], bq, sfb, alpha)
        full_rms = TOL.rms(OG.nvfp4_gemm_f64(aq, sfa, bq, sfb, alpha)) if M <= 128 else None
        ok, worst, nbad = TOL.check_bf16(host_bf16_bits(out)[rows], want, rms_ref=full_rms)
        assert ok, (M, N, K, worst, nbad)


def test_noalloc_mxfp4_and_refusal():
    lib = bs.load()
    M, N, K = 96, 512, 1024
    aq, sfa, bq, sfb = mxfp4_problem(M, N, K, 320)
    daq, dsfa, dbq, dsfb = dev_u8(aq), dev_u8(sfa), dev_u8(bq), dev_u8(sfb)
    ref = bs.gemm(daq, dsfa, dbq, dsfb, None, fmt="mxfp4")
    out = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    assert _noalloc(lib, 1, daq, dsfa, dbq, dsfb, None, out, M, N, K) == 0
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    # more partials than the static scratch holds: refused before any launch
    M2 = 1024
    assert lib.fp4_gemm_workspace_size(0, M2, 4096, 7168) > lib.fp4_gemm_noalloc_max_workspace()
    big = torch.empty((M2, 4096), dtype=torch.bfloat16, device=DEV)
    a16 = torch.empty((M2, 3584), dtype=torch.uint8, device=DEV)
    s16 = torch.empty((M2, 448), dtype=torch.uint8, device=DEV)
    b16 = torch.empty((4096, 3584), dtype=torch.uint8, device=DEV)
    t16 = torch.empty((4096, 448), dtype=torch.uint8, device=DEV)
    st = _noalloc(lib, 0, a16, s16, b16, t16, None, big, M2, 4096, 7168)
    assert st == WORKSPACE and "static scratch" in lib.bsfp4_last_error().decode()

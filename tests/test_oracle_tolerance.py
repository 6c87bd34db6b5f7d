"""Pins of the acceptance rule (oracle/tolerance.py).

The rule is the one the project states for every GEMM and MoE output,

    |D - Dref| <= 8e-3 * |Dref| + 1e-3 * rms(Dref),   rms over the whole Dref,

where Dref is the float64 result rounded once to bf16 (the "Alpha epilogue
bug" section of "perf(gemm): optimize SM103 CuTe DSL mm_fp4 kernel" fixes the
single conversion).  The pages print no tolerance, so the constants are pinned
by their definition only; what these tests pin is that the code implements
that definition: the bound is recomputed here in exact rational arithmetic
(fractions.Fraction of the decimal constants), bf16 neighbours are taken from
the sorted grid of every finite bf16 value, and each test is built so that a plausible slip
(inverted inequality, a wrong constant, rms of D instead of Dref, a missing
abs, comparing Dref with itself, a non-finite value slipping through, an
ignored rms override) fails at least one of them.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest

from oracle import tolerance as TOL

REL = Fraction(8, 1000)
ABS = Fraction(1, 1000)


def _bound(r: float, rms: float) -> Fraction:
    return REL * abs(Fraction(r)) + ABS * Fraction(rms)


def _bf16_val(bits: int) -> float:
    return float(np.array([bits << 16], np.uint32).view(np.float32)[0])


def _bf16_bits(v: float) -> int:
    b = int(np.array([v], np.float32).view(np.uint32)[0])
    assert b & 0xFFFF == 0, "value must be a bf16"
    return b >> 16


def _rms_exact(vals) -> float:
    return float(np.sqrt(np.mean(np.square(np.asarray(vals, np.float64)))))


@pytest.mark.parametrize("r", [1.0, -3.75, 250.0, 1.0e-3, 0.0, -0.0])
@pytest.mark.parametrize("rms", [0.5, 1.0, 10.0])
def test_bound_edge_float64(r, rms):
    """Just inside the bound passes, just outside fails, on both sides of Dref."""
    b = float(_bound(r, rms))
    for sign in (1.0, -1.0):
        d_in = r + sign * b * (1 - 1e-9)
        d_out = r + sign * b * (1 + 1e-9)
        ok, worst, nbad = TOL.check_f64([d_in], [r], rms_ref=rms)
        assert ok and nbad == 0 and worst <= 1.0
        ok, worst, nbad = TOL.check_f64([d_out], [r], rms_ref=rms)
        assert not ok and nbad == 1 and worst > 1.0


def _finite_bf16_sorted():
    """Every finite bf16 bit pattern, -0 dropped, sorted by value."""
    bits = np.arange(0x10000, dtype=np.uint32)
    with np.errstate(invalid="ignore"):   # NaN patterns are dropped below
        vals = (bits << 16).view(np.float32).astype(np.float64)
    keep = np.isfinite(vals) & (bits != 0x8000)
    bits, vals = bits[keep], vals[keep]
    order = np.argsort(vals, kind="stable")
    return bits[order].astype(np.uint16), vals[order]


_BITS, _VALS = _finite_bf16_sorted()


@pytest.mark.parametrize("r", [1.0, 3.703125, -250.0, 0.0009765625, 0.0, 57344.0])
@pytest.mark.parametrize("rms", [0.25, 1.0, 10.0, 700.0])
def test_bound_edge_one_bf16_step(r, rms):
    """Walk the bf16 grid away from Dref: the last value within the exact
    bound passes, the next bf16 value (one step further) fails."""
    rb = np.uint16(_bf16_bits(r))
    i0 = int(np.searchsorted(_VALS, r))
    assert _VALS[i0] == r
    b = _bound(r, rms)
    for direction in (+1, -1):
        i = i0
        while abs(Fraction(float(_VALS[i + direction])) - Fraction(r)) <= b:
            i += direction
        last_in, first_out = _BITS[i], _BITS[i + direction]
        assert last_in != first_out
        for cand, expect in ((first_out, False), (last_in, True)):
            err = abs(Fraction(_bf16_val(int(cand))) - Fraction(r))
            # skip a value whose exact distance sits within float64 rounding of the bound
            if abs(err - b) < b * Fraction(1, 10**12):
                continue
            ok, _, _ = TOL.check_bf16(np.array([cand], np.uint16), np.array([rb], np.uint16), rms_ref=rms)
            assert ok is expect, (r, rms, direction, hex(int(cand)))


def test_zero_reference_uses_only_the_rms_term():
    ref = np.array([0.0, 0.0, 0.0, 2.0])       # rms = 1 exactly
    assert _rms_exact(ref) == 1.0
    ok, _, _ = TOL.check_f64([0.99e-3, 0, 0, 2.0], ref)
    assert ok
    ok, _, nbad = TOL.check_f64([1.01e-3, 0, 0, 2.0], ref)
    assert not ok and nbad == 1
    ok, _, _ = TOL.check_f64([-1.01e-3, 0, 0, 2.0], ref)
    assert not ok


def test_default_rms_is_that_of_the_reference_not_of_d():
    # rms(Dref) = sqrt(50) = 7.0711; rms(D) is larger because
    # D's large element sits 0.08 above Dref's (within its own bound 0.081)
    ref = np.array([0.0, 10.0])
    rms_ref = _rms_exact(ref)
    d_ok = np.array([7.0e-3, 10.08])
    d_bad = np.array([7.1e-3, 10.08])
    assert 7.0e-3 < float(ABS * Fraction(rms_ref)) < 7.1e-3 < float(ABS * Fraction(_rms_exact(d_bad)))
    assert TOL.check_f64(d_ok, ref)[0]
    ok, _, nbad = TOL.check_f64(d_bad, ref)
    assert not ok and nbad == 1


def test_rms_override_for_sampled_rows():
    """Sampled rows are checked with the rms of the whole output passed in."""
    ref_rows = np.array([0.0, 1.0, -1.0, 0.5])          # rms of the sample 0.75
    d = np.array([5e-3, 1.0, -1.0, 0.5])
    assert not TOL.check_f64(d, ref_rows)[0]             # bound at 0: 7.5e-4
    assert TOL.check_f64(d, ref_rows, rms_ref=10.0)[0]   # bound at 0: 1e-2
    assert not TOL.check_f64(d, ref_rows, rms_ref=4.0)[0]
    with pytest.raises(ValueError):
        TOL.check_f64(d, ref_rows, rms_ref=float("nan"))
    with pytest.raises(ValueError):
        TOL.check_f64(d, ref_rows, rms_ref=-1.0)


def test_non_finite_values():
    nan, inf = float("nan"), float("inf")
    # non-finite D against a finite reference
    assert not TOL.check_f64([nan, 2.0], [1.0, 2.0])[0]
    assert not TOL.check_f64([inf, 2.0], [1.0, 2.0])[0]
    assert not TOL.check_f64([-inf, 2.0], [1.0, 2.0])[0]
    # non-finite reference against a finite D: must not pass silently
    ok, worst, nbad = TOL.check_f64([1.0, 2.0], [nan, 2.0])
    assert not ok and nbad == 1 and worst == inf
    assert not TOL.check_f64([1.0, 2.0], [inf, 2.0])[0]
    # identical non-finite values pass; a different one does not
    assert TOL.check_f64([nan, 2.0], [nan, 2.0])[0]
    assert TOL.check_f64([inf, 2.0], [inf, 2.0])[0]
    assert not TOL.check_f64([-inf, 2.0], [inf, 2.0])[0]
    assert not TOL.check_f64([nan, 2.0], [inf, 2.0])[0]
    # an infinite reference element must not widen every other element's bound
    assert not TOL.check_f64([inf, 0.5], [inf, 0.0])[0]
    # bf16 bit patterns: 0x7FC0 NaN, 0x7F80 +inf
    assert not TOL.check_bf16(np.array([0x7FC0], np.uint16), np.array([0x3F80], np.uint16))[0]
    assert not TOL.check_bf16(np.array([0x3F80], np.uint16), np.array([0x7FC0], np.uint16))[0]
    assert not TOL.check_bf16(np.array([0x7F80], np.uint16), np.array([0x3F80], np.uint16))[0]


def test_counts_and_worst_ratio():
    ref = np.array([1.0, 2.0, 4.0, 0.0])
    rms = _rms_exact(ref)
    b = [float(_bound(v, rms)) for v in ref]
    d = ref + np.array([0.5 * b[0], 3.0 * b[1], -2.0 * b[2], 0.0])
    ok, worst, nbad = TOL.check_f64(d, ref)
    assert not ok and nbad == 2
    assert worst == pytest.approx(3.0, rel=1e-9)
    # identical outputs: ok, ratio 0
    assert TOL.check_f64(ref, ref) == (True, 0.0, 0)
    # the bound is inclusive: an all-zero output (bound 0, error 0) passes
    assert TOL.check_f64(np.zeros(4), np.zeros(4)) == (True, 0.0, 0)
    ok, worst, nbad = TOL.check_f64([0.0, 1e-300], np.zeros(2))
    assert not ok and nbad == 1 and worst == float("inf")


def test_shape_mismatch_and_empty():
    with pytest.raises(ValueError):
        TOL.check_f64([1.0, 2.0], [1.0])
    assert TOL.check_f64(np.zeros((0, 3)), np.zeros((0, 3))) == (True, 0.0, 0)

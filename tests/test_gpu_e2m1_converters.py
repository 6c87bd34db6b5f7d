"""Exhaustive and dense sweeps of the kernels' E2M1 converters against the
oracle's encoder (bit for bit).

The quantisers and the fused SiLU-mul + MXFP4 epilogue produce E2M1 codes with
gfx950's v_cvt_scalef32_pk_fp4_* instructions; the rule they must follow is the
encoder of the oracle (nearest E2M1 value, ties to the even code, saturation at
6, sign bit kept), this project's reading of the per-block routine that the
vLLM `sm103` branch comparison page calls (`cvt_fp16_to_fp4_sm103`) but does not
print.  The library exports those exact device routines through
bsfp4_e2m1_convert; these tests feed them:
  * the bf16 form: all 65,536 bf16 patterns except NaN, at several E8M0 scales;
  * the binary32 form (scale 1): every E2M1 grid point and midpoint, +-1..3
    ulp around each, both signs, +-0, subnormals, +-inf, huge values, and a
    dense random sweep of binary32 patterns;
  * the binary32 form with an E8M0 scale (the fused epilogue): the same
    special values moved by the scale, and random patterns.
Expected codes come from oracle.formats.e2m1_encode of the exact quotient.
"""
import numpy as np
import pytest
import torch

import block_scaled_fp4_e2m1_amd as bs
from oracle.formats import e2m1_encode

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
MIDPOINTS = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]


def _expected_pairs(vals64):
    """Packed expected bytes for a flat array of exact values (pairs in order)."""
    with np.errstate(over="ignore"):    # quotients beyond binary32 become inf: code 7, as their value
        codes = e2m1_encode(vals64)     # rounds to binary32 first: exact below the overflow
    return (codes[0::2] & 0xF) | ((codes[1::2] & 0xF) << 4)


def _pad8(a, fill):
    n = (-len(a)) % 8
    return np.concatenate([a, np.full(n, fill, a.dtype)]) if n else a


def _run_f32(vals32, scodes=None):
    vals32 = np.ascontiguousarray(vals32, np.float32)
    t = torch.from_numpy(vals32).to(DEV)
    s = None if scodes is None else torch.from_numpy(np.ascontiguousarray(scodes, np.uint8)).to(DEV)
    return bs.e2m1_convert(t, s).cpu().numpy()


def _report(got, want, inputs):
    bad = np.nonzero(got != want)[0]
    if bad.size:
        i = bad[0]
        return f"{bad.size} mismatches; first pair {i}: inputs {inputs[2 * i]!r}, {inputs[2 * i + 1]!r} " \
               f"got {got[i]:#04x} want {want[i]:#04x}"
    return ""


def _special_f32():
    v = []
    f = np.float32
    for p in GRID + MIDPOINTS:
        x = f(p)
        v.append(x)
        up, dn = x, x
        for _ in range(3):
            up = np.nextafter(up, f(np.inf))
            dn = np.nextafter(dn, f(-np.inf))
            v += [up, dn]
    v += [f(0.0), f(np.finfo(np.float32).tiny), f(np.finfo(np.float32).max), f(np.inf), f(1e30), f(7.0),
          f(6.5), f(5.999999), f(100.0)]
    sub = np.array([1, 2, 3, 0x3FFFFF, 0x400000, 0x7FFFFF], np.uint32).view(np.float32)
    v += list(sub)
    v = np.array(v, np.float32)
    v = np.concatenate([v, -v])                  # both signs, incl. -0 and -inf
    return v


def test_f32_form_special_values():
    v = _pad8(_special_f32(), np.float32(0.0))
    # every special value in both slots of a pair: the value list and its reversal
    vals = np.concatenate([v, v[::-1]])
    got = _run_f32(vals)
    want = _expected_pairs(vals.astype(np.float64))
    assert not _report(got, want, vals), _report(got, want, vals)


def test_f32_form_dense_random():
    rng = np.random.default_rng(7001)
    # exponents around the E2M1 range (2^-12 .. 2^4), every sign and mantissa
    n = 1 << 20
    e = rng.integers(127 - 12, 127 + 5, n, dtype=np.uint32)
    m = rng.integers(0, 1 << 23, n, dtype=np.uint32)
    s = rng.integers(0, 2, n, dtype=np.uint32)
    near = ((s << 31) | (e << 23) | m).view(np.float32)
    # and unrestricted finite patterns
    anyp = rng.integers(0, 1 << 32, 1 << 18, dtype=np.uint64).astype(np.uint32).view(np.float32)
    anyp = anyp[np.isfinite(anyp)]
    vals = _pad8(np.concatenate([near, anyp]), np.float32(0.0))
    got = _run_f32(vals)
    want = _expected_pairs(vals.astype(np.float64))
    assert not _report(got, want, vals), _report(got, want, vals)


def _all_bf16_non_nan():
    bits = np.arange(0x10000, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    return bits[~np.isnan(f)].astype(np.uint16)


@pytest.mark.parametrize("scode", [0, 1, 2, 100, 124, 126, 127, 128, 129, 133, 200, 253, 254])
def test_bf16_form_every_pattern(scode):
    bits = _pad8(_all_bf16_non_nan(), np.uint16(0))
    pairs = bits.size // 2
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    sc = torch.full((pairs,), scode, dtype=torch.uint8, device=DEV)
    got = bs.e2m1_convert(t, sc).cpu().numpy()
    vals = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    want = _expected_pairs(np.ldexp(vals, 127 - scode))
    assert not _report(got, want, vals), f"scale code {scode}: " + _report(got, want, vals)


def test_bf16_form_mixed_scales_per_pair():
    """A different scale code for every pair, exercising all four byte slots."""
    rng = np.random.default_rng(7002)
    bits = _all_bf16_non_nan()
    bits = _pad8(bits[rng.permutation(bits.size)], np.uint16(0))
    pairs = bits.size // 2
    sc = rng.integers(0, 255, pairs, dtype=np.uint8)
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    got = bs.e2m1_convert(t, torch.from_numpy(sc).to(DEV)).cpu().numpy()
    vals = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    want = _expected_pairs(np.ldexp(vals, 127 - np.repeat(sc.astype(np.int64), 2)))
    assert not _report(got, want, vals), _report(got, want, vals)


@pytest.mark.parametrize("scode", [0, 1, 120, 126, 127, 128, 131, 254])
def test_f32_form_with_e8m0_scale(scode):
    """The fused epilogue's form: special values moved onto the scale's grid
    (exactly: power-of-two multiples), plus random patterns."""
    base = _special_f32().astype(np.float64)
    with np.errstate(over="ignore"):
        moved = np.ldexp(base, scode - 127).astype(np.float32)  # exact unless it leaves binary32's range
    rng = np.random.default_rng(7100 + scode)
    e = np.clip(rng.integers(scode - 12, scode + 5, 1 << 16), 1, 254).astype(np.uint32)
    m = rng.integers(0, 1 << 23, 1 << 16, dtype=np.uint32)
    s = rng.integers(0, 2, 1 << 16, dtype=np.uint32)
    rnd = ((s << 31) | (e << 23) | m).view(np.float32)
    vals = _pad8(np.concatenate([moved, rnd]), np.float32(0.0))
    sc = np.full(vals.size // 2, scode, np.uint8)
    got = _run_f32(vals, sc)
    want = _expected_pairs(np.ldexp(vals.astype(np.float64), 127 - scode))
    assert not _report(got, want, vals), f"scale code {scode}: " + _report(got, want, vals)

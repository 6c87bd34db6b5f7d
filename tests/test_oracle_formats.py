"""Pins for oracle/formats.py: decode tables and encoders.

Each check compares the oracle with something other than itself: the
hand-written fixture of format landmarks, torch's float8 views and casts
(library routines), brute-force nearest-point searches, or exact rational
arithmetic.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F


@pytest.fixture(scope="module")
def fmt(golden_dir):
    with open(os.path.join(golden_dir, "formats.json")) as f:
        return json.load(f)


# ---------------------------------------------------------------- tables

def test_e2m1_table_matches_fixture(fmt):
    mags = fmt["e2m1_magnitudes_by_code_0_to_7"]
    for c in range(8):
        assert F.E2M1_TABLE[c] == mags[c]
        assert F.E2M1_TABLE[c | 8] == -mags[c]
    assert math.copysign(1.0, F.E2M1_TABLE[8]) == -1.0  # code 8 is -0.0
    assert F.E2M1_MAX == fmt["e2m1_max"] == max(mags)


def test_e4m3_table_matches_torch_and_fixture(fmt):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both_nan = np.isnan(ref) & np.isnan(F.E4M3_TABLE)
    assert np.all(both_nan | (ref == F.E4M3_TABLE))
    assert [c for c in range(256) if math.isnan(F.E4M3_TABLE[c])] == [
        int(h, 16) for h in fmt["e4m3_nan_codes"]]
    for lm in fmt["e4m3_landmarks"]:
        assert F.E4M3_TABLE[int(lm["code"], 16)] == lm["value"], lm
    assert np.nanmax(F.E4M3_TABLE) == fmt["e4m3_max"] == F.E4M3_MAX


def test_e8m0_table_matches_torch_and_fixture(fmt):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.isnan(ref[255]) and np.isnan(F.E8M0_TABLE[255])
    assert np.array_equal(ref[:255], F.E8M0_TABLE[:255])
    for lm in fmt["e8m0_landmarks"]:
        assert F.E8M0_TABLE[lm["code"]] == 2.0 ** lm["value_log2"]


# ---------------------------------------------------------------- E2M1 encoder

def _e2m1_brute(y: float, mags) -> int:
    """Nearest of the 8 magnitudes, ties to the even code, saturating at 6."""
    a = abs(Fraction(y))
    best = None
    for c, m in enumerate(mags):
        d = abs(a - Fraction(m))
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    code = best[1]
    return code | (8 if math.copysign(1.0, y) < 0 else 0)


def _e2m1_probe_values():
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    pts = []
    for lo, hi in zip(mags[:-1], mags[1:]):
        mid = np.float32((lo + hi) / 2)
        pts += [mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(10))]
    pts += [np.float32(m) for m in mags]
    pts += [np.float32(6.5), np.float32(7.999), np.float32(1e30), np.float32(1e-30)]
    rng = np.random.default_rng(7)
    pts += list(rng.uniform(0, 8, 4000).astype(np.float32))
    pts += list(np.linspace(0, 7, 7001, dtype=np.float32))
    v = np.array(pts, dtype=np.float32)
    return np.concatenate([v, -v])


def test_e2m1_encoder_is_nearest_even(fmt):
    mags = fmt["e2m1_magnitudes_by_code_0_to_7"]
    y = _e2m1_probe_values()
    got = F.e2m1_encode(y)
    want = np.array([_e2m1_brute(float(t), mags) for t in y], dtype=np.uint8)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(y[i]), int(got[i]), int(want[i])) for i in bad[:10]]


def test_e2m1_roundtrip_and_sign_of_zero():
    for c in range(16):
        assert F.e2m1_encode(np.float32(F.E2M1_TABLE[c]))[()] == c
    assert F.e2m1_encode(np.float32(-0.0))[()] == 8
    assert F.e2m1_encode(np.float32(-0.2))[()] == 8
    assert F.e2m1_encode(np.float32(0.2))[()] == 0


def test_e2m1_encoder_monotone():
    y = np.linspace(-7, 7, 20001, dtype=np.float32)
    vals = F.E2M1_TABLE[F.e2m1_encode(y)]
    assert np.all(np.diff(vals) >= 0)


# ---------------------------------------------------------------- E4M3 encoder

def _e4m3_probe_values():
    pos = F.E4M3_TABLE[:0x7F]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    pts = [mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9)),
           pos.astype(np.float32)]
    rng = np.random.default_rng(11)
    pts.append(np.exp2(rng.uniform(-12, 8.85, 20000)).astype(np.float32))
    pts.append(np.float32([0.0, 2.0 ** -10, 2.0 ** -11, 1e-12, 447.9, 448.0, 455.99, 463.99]))
    s = np.concatenate(pts)
    return s[s < 464]


def test_e4m3_encoder_matches_torch_cast():
    s = _e4m3_probe_values()
    got = F.e4m3_encode_satfinite(s)
    ref = torch.from_numpy(s).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(s[i]), int(got[i]), int(ref[i])) for i in bad[:10]]


def test_e4m3_encoder_saturates():
    s = np.float32([448.0, 464.0, 465.0, 1000.0, 3.0e38])
    assert np.all(F.e4m3_encode_satfinite(s) == 0x7E)


def test_e4m3_roundtrip():
    for c in range(0x7F):
        assert F.e4m3_encode_satfinite(np.float32(F.E4M3_TABLE[c]))[()] == c


# ---------------------------------------------------------------- E8M0 encoder

def _e8m0_brute(s: float) -> int:
    for c in range(255):
        if math.ldexp(1.0, c - 127) >= s:
            return c
    return 254


def test_e8m0_ceil_brute_force():
    rng = np.random.default_rng(5)
    s = np.concatenate([
        np.exp2(rng.uniform(-140, 127, 5000)).astype(np.float32),
        np.float32([0.0, 1.0, 2.0, 0.5, 1.0000001, 0.99999994, 2.0 ** -127, 2.0 ** -128,
                    2.0 ** -149, 3.0, 6.0, 7.0 / 6.0]),
    ])
    got = F.e8m0_encode_ceil(s)
    want = np.array([_e8m0_brute(float(v)) for v in s], dtype=np.uint8)
    assert np.array_equal(got, want)


# ---------------------------------------------------------------- bf16 from float64

def _bf16_exact(x: float) -> float:
    """RNE of x to 8 significant bits (exact rationals), subnormals at 2^-133."""
    if x == 0:
        return x
    f = Fraction(x)
    a = abs(f)
    e = math.floor(math.log2(a))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = Fraction(2) ** (max(e, -126) - 7)
    r = round(a / q) * q          # Python rounds Fraction halves to even
    if r >= Fraction(2) ** 128:
        return math.copysign(math.inf, x)
    return math.copysign(float(r), x)


def test_bf16_rne_from_f64_exact():
    rng = np.random.default_rng(3)
    xs = list(rng.standard_normal(3000) * np.exp2(rng.uniform(-30, 30, 3000)))
    # exact ties and near-ties on the bf16 grid
    for base in [1.0, 1.5, 3.0, 1000.0, 2.0 ** -120, 2.0 ** -130]:
        half = 2.0 ** (max(math.floor(math.log2(base)), -126) - 8)  # half the bf16 spacing
        for k in range(8):
            mid = base + (2 * k + 1) * half
            xs += [mid, -mid, np.nextafter(mid, 0), np.nextafter(mid, 10)]
    xs += [0.0, -0.0, 3.3e38, 3.4e38, 2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -135]
    xs = np.array(xs, dtype=np.float64)
    got = F.bf16_bits_to_f64(F.bf16_rne_from_f64(xs))
    want = np.array([_bf16_exact(float(v)) for v in xs])
    assert np.array_equal(got, want)


def test_bf16_rne_matches_torch_from_f32():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal(20000) * 50).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(F.bf16_rne_from_f64(x.astype(np.float64)), ref)


def test_nibble_order():
    # element 2j in the low nibble (vLLM sm103 page: the first elements of a
    # thread's vector land in the low bits of the packed word)
    packed = F.pack_nibbles(np.array([[1, 2, 3, 4]], dtype=np.uint8))
    assert packed.tolist() == [[0x21, 0x43]]
    assert F.unpack_nibbles(packed).tolist() == [[1, 2, 3, 4]]

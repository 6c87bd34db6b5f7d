"""Acceptance rule for floating-point outputs (CPU oracle).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

A GPU output D (bf16) passes against the float64 result rounded once to
bf16, Dref, when every element satisfies

    |D - Dref| <= 8e-3 * |Dref| + 1e-3 * rms(Dref)

with rms taken over the whole output.  Derivation: the GPU path sums exact
products in binary32 (relative error ~ sqrt(K) * 2**-24, negligible) and
rounds once to bf16; two independent bf16 roundings of nearly equal values
differ by at most one bf16 step, which is below 2**-7 = 7.8e-3 of the
value's magnitude; the rms term absorbs cancellation near zero, where the
binary32 summation error is no longer small relative to |Dref|.

Non-finite values lie outside that rule (the inputs the pages describe are
finite).  An element whose Dref is NaN or infinite passes only when D holds
the same value there (both NaN, or the same infinity); a non-finite D
against a finite Dref fails; rms(Dref) is taken over the finite entries, so
a stray infinity in Dref cannot widen the bound of every other element.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_bits_to_f64

REL = 8e-3
ABS_RMS = 1e-3


def rms(x) -> float:
    x = np.asarray(x, dtype=np.float64)
    return float(np.sqrt(np.mean(x * x))) if x.size else 0.0


def check_bf16(D_bits, Dref_bits, rms_ref: float | None = None):
    """Return (ok, worst_ratio, n_bad) for bf16 outputs given as uint16 bits.

    rms_ref may be passed in when D covers only sampled rows of a larger
    output; by default it is the rms of Dref itself.
    """
    d = bf16_bits_to_f64(D_bits)
    r = bf16_bits_to_f64(Dref_bits)
    return check_f64(d, r, rms_ref)


def check_f64(d, r, rms_ref: float | None = None):
    """Return (ok, worst_ratio, n_bad): ok when every element obeys the rule.

    worst_ratio is max |D - Dref| / bound over the finite elements (inf where
    an element fails with a zero bound or a non-finite mismatch).
    """
    d = np.asarray(d, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    if d.shape != r.shape:
        raise ValueError(f"shape mismatch {d.shape} vs {r.shape}")
    r_fin = np.isfinite(r)
    d_fin = np.isfinite(d)
    if rms_ref is None:
        rms_ref = rms(r[r_fin])
    elif not (np.isfinite(rms_ref) and rms_ref >= 0):
        raise ValueError(f"rms_ref must be finite and >= 0, got {rms_ref}")
    both = r_fin & d_fin
    rr = np.where(both, r, 0.0)
    dd = np.where(both, d, 0.0)
    bound = REL * np.abs(rr) + ABS_RMS * rms_ref
    err = np.abs(dd - rr)
    # a non-finite reference must be matched exactly (NaN by NaN, inf by the same inf)
    same_nonfinite = (~r_fin) & ((np.isnan(r) & np.isnan(d)) | (np.isinf(r) & (d == r)))
    bad = np.where(both, err > bound, ~same_nonfinite)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, err / bound, np.where(err > 0, np.inf, 0.0))
    ratio = np.where(both, ratio, np.where(bad, np.inf, 0.0))
    worst = float(np.max(ratio)) if ratio.size else 0.0
    return (not bool(np.any(bad))), worst, int(np.count_nonzero(bad))

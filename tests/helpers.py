"""Test-side helpers: tolerance units and exact-rounding references.

Nothing here is shared with the GPU library; the exact-rounding references use
Python's Fraction/Decimal arithmetic, a method independent of the oracle's C code.
"""
from __future__ import annotations

import bisect
import math
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np

getcontext().prec = 60


def ulp_bf16(v):
    """bf16 unit in the last place at the (exact) value v: 2^(max(floor(log2|v|), -126) - 7); 2^-133 at 0."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, e2 = np.frexp(np.where(a > 0, a, 1.0))  # a = f * 2^e2, f in [0.5, 1)
    e = (e2 - 1).astype(np.float64)
    e = np.maximum(e, -126.0)
    u = np.ldexp(1.0, (e - 7).astype(np.int64))
    return np.where(a > 0, u, 2.0 ** -133)


def bf16_bits_to_f64(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def within_bf16_ulps(y_bits, y_ref, n_ulps=2.0):
    """Per-element |y - y_ref| <= n_ulps * ulp_bf16(y_ref); returns (ok_mask, err_in_ulps)."""
    y = bf16_bits_to_f64(y_bits)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    u = ulp_bf16(y_ref)
    err = np.abs(y - y_ref) / u
    return err <= n_ulps, err


FP32_FLOOR = 2.0 ** -24  # one fp32 rounding, relative


def parity_bar(y_bits, y_ref, mass, n_ulps=2.0):
    """The projection's per-element bar: |y - y_ref| <= n_ulps * ulp_bf16(y_ref), except where the exact
    value has cancelled below what an fp32 accumulation of the terms can resolve -- then |y - y_ref|
    must lie within one fp32 rounding of the terms' absolute sum, 2^-24 * sum_k |q s x| (`mass`).
    Returns (ok_mask, err_in_ulps, misses): misses = the outputs beyond n_ulps ulps that pass only by
    that floor (reported per workload)."""
    y = bf16_bits_to_f64(y_bits)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    d = np.abs(y - y_ref)
    err = d / ulp_bf16(y_ref)
    in_ulps = err <= n_ulps
    ok = in_ulps | (d <= FP32_FLOOR * np.asarray(mass, dtype=np.float64))
    return ok, err, int(np.sum(ok & ~in_ulps))


def rn32(x) -> np.float32:
    """Correctly round an exact value (Fraction, Decimal, int or float) to binary32, ties to even."""
    f = Fraction(x)
    if f == 0:
        return np.float32(0.0)
    approx = np.float32(float(f))
    if np.isinf(approx):
        return approx
    cands = [np.nextafter(approx, np.float32(-np.inf)), approx, np.nextafter(approx, np.float32(np.inf))]
    best, bestd = None, None
    for c in cands:
        if not np.isfinite(c):
            continue
        d = abs(Fraction(float(c)) - f)
        if bestd is None or d < bestd or (d == bestd and (int(np.float32(c).view(np.uint32)) & 1) == 0):
            best, bestd = c, d
    # overflow: beyond max finite + half ulp rounds to infinity
    fmax = Fraction(float(np.finfo(np.float32).max))
    half = Fraction(2) ** 103  # half ulp at the top binade (ulp 2^104)
    if abs(f) >= fmax + half:
        return np.float32(math.copysign(np.inf, float(f)))
    return np.float32(best)


def exp_rn32(x: float) -> np.float32:
    return rn32(Decimal(float(x)).exp())


def ln_rn32(x: float) -> np.float32:
    return rn32(Decimal(float(x)).ln())


_BF16_POS = None


def _bf16_positive_table():
    global _BF16_POS
    if _BF16_POS is None:
        pats = np.arange(0, 0x7F81, dtype=np.uint16)  # +0 ... +inf
        _BF16_POS = [Fraction(float(v)) if np.isfinite(v) else None for v in bf16_bits_to_f64(pats)]
    return _BF16_POS


def bf16_round_by_search(v: float) -> int:
    """RNE of a double to bf16 by searching the ordered table of bf16 values (independent of scaling)."""
    if math.isnan(v):
        return 0x7FC0
    sign = 0x8000 if math.copysign(1.0, v) < 0 else 0
    a = Fraction(abs(v)) if math.isfinite(v) else None
    if a is None:
        return sign | 0x7F80
    table = _bf16_positive_table()
    finite = table[:0x7F80]
    i = bisect.bisect_right(finite, a) - 1  # largest pattern with value <= a
    if finite[i] == a:
        return sign | i
    lo = i
    if lo + 1 >= 0x7F80:
        hi_val = Fraction(2) ** 128  # the overflow boundary behaves like the next grid point
    else:
        hi_val = finite[lo + 1]
    dlo, dhi = a - finite[lo], hi_val - a
    if dlo < dhi or (dlo == dhi and lo % 2 == 0):
        return sign | lo
    return sign | (lo + 1 if lo + 1 < 0x7F80 else 0x7F80)

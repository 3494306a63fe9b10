"""The oracle's LOG32 is the correctly rounded ln over the whole domain the logprob's fold uses.

The fold takes the logarithm of S, the sum of the row's exponentials: the maximum contributes exactly
1 and every other term is at most 1, so S lies in [1, V] and V <= 2^31.  The oracle computes LOG32 as
(float)logl(x): the long-double logarithm (64-bit significand) rounded once more to binary32.  Two
roundings can differ from one correct rounding only where the long-double value lies within the
long-double logarithm's own error of a binary32 rounding boundary (a midpoint between two floats).
This test runs over every binary32 x in [1, 2^31] (260,046,849 values, in chunks):
  * numpy's long-double log (the same libm logl, evaluated independently of the oracle's C code) is
    rounded to binary32 and compared with the oracle's value for every x;
  * every x whose long-double logarithm lies within 2^-24 binary32 ulps of a midpoint -- a margin
    some 2^15 times the long-double error -- is decided exactly: RN32 of a 60-digit decimal ln.
So the oracle's LOG32 equals RN32(ln x) for every x the fold can see, without trusting the double
rounding anywhere it could matter.
"""
import numpy as np
import pytest

import oracle
from tests.helpers import ln_rn32

pytestmark = pytest.mark.slow

LO, HI = 0x3F800000, 0x4F000000  # bit patterns of 1.0 and 2^31
CHUNK = 1 << 24
MARGIN = 2.0 ** -24              # in binary32 ulps of the result


def test_oracle_log32_is_correctly_rounded_on_the_fold_domain():
    assert np.longdouble(1) + np.longdouble(2.0 ** -63) != np.longdouble(1), "needs an 80-bit long double"
    total = near = 0
    for start in range(LO, HI + 1, CHUNK):
        n = min(CHUNK, HI + 1 - start)
        xb = np.arange(start, start + n, dtype=np.uint32)
        x = xb.view(np.float32)
        y = np.log(x.astype(np.longdouble))
        f = y.astype(np.float32)
        got = oracle.log32_bits(start, n)
        assert np.array_equal(got.view(np.uint32), f.view(np.uint32)), f"chunk at {start:#x}"
        # distance of y from the midpoint on its side of f, in ulps of f (f > 0 here except at x = 1)
        up = np.nextafter(f, np.float32(np.inf))
        dn = np.nextafter(f, np.float32(-np.inf))
        fl = f.astype(np.longdouble)
        side_up = y >= fl
        mid = np.where(side_up, (fl + up.astype(np.longdouble)) / 2, (fl + dn.astype(np.longdouble)) / 2)
        ulp = np.where(side_up, up.astype(np.longdouble) - fl, fl - dn.astype(np.longdouble))
        dist = np.abs(y - mid) / ulp
        suspects = np.nonzero(dist < MARGIN)[0]
        for i in suspects:
            assert f[i] == ln_rn32(float(x[i])), f"x = {float(x[i])!r}: oracle {f[i]!r}"
        near += suspects.size
        total += n
    assert total == HI - LO + 1
    print(f"LOG32 over [1, 2^31]: {total} values, {near} decided by the decimal reference")

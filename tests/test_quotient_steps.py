"""Exact-arithmetic check of the division-free quotient the INT4 code uses.

The device computes fl(x / s) for an fp16 group scale s as: y = fl(1/s) from
the hardware reciprocal (within one ulp) and one residual step; q0 = fl(x y);
r = x - s q0 with one fma; q = fl(q0 + r y) (Markstein's correction step).
The code rint(q) must equal rint of the correctly rounded quotient, so q must
equal fl(x / s) wherever rint can change, at the midpoints (k + 1/2) s.  The
steps commute with scaling by powers of two, so every fp16 significand at one
exponent covers every normal and subnormal fp16 scale.  This module redoes
the steps in rational arithmetic with round-to-nearest-even to fp32.
"""
import math
from fractions import Fraction as F

import pytest


def _binade(a: F) -> int:
    e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
    while F(2) ** e > a:
        e -= 1
    while F(2) ** (e + 1) <= a:
        e += 1
    return e


def _ulp(v: F) -> F:
    return F(2) ** (_binade(abs(v)) - 23)


def _rn(v: F) -> F:
    """nearest fp32 to v (ties to even), normal range"""
    if v == 0:
        return F(0)
    u = _ulp(v)
    n = abs(v) / u
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > F(1, 2) or (rem == F(1, 2) and fl % 2 == 1):
        fl += 1
    return (1 if v > 0 else -1) * fl * u


def _recip(s: F, y0: F) -> F:
    return _rn(y0 + _rn(1 - s * y0) * y0)


def _quot(x: F, s: F, y: F):
    q0 = _rn(x * y)
    r_exact = x - s * q0
    r = _rn(r_exact) if r_exact != 0 else F(0)
    return _rn(q0 + r * y) if q0 + r * y != 0 else F(0), r == r_exact


@pytest.mark.parametrize("block", range(8))
def test_reciprocal_and_quotient_exact(block):
    for m in range(128 * block, 128 * block + 128):
        s = F(1024 + m, 1024)                    # fp16 significand 1.m
        t = _rn(1 / s)
        u = _ulp(t)
        for d in (-2, -1, 0, 1, 2):              # any start within two ulps
            assert _recip(s, t + d * u) == t, (m, d)
        for k in range(16):
            xm = (k + F(1, 2)) * s                # midpoint, exact in fp32
            uu = _ulp(xm)
            for j in range(-4, 5):
                x = xm + j * uu
                q, exact_r = _quot(x, s, t)
                assert exact_r, (m, k, j)
                assert q == _rn(x / s), (m, k, j)

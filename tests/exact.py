"""Exact-arithmetic helpers for pinning the oracle (pure Python, no numpy rounding).

Independent of numpy's float conversions: IEEE round-to-nearest-even written
out from its definition on Fractions.
"""

from __future__ import annotations

import math
from fractions import Fraction

# (significand bits incl. the leading one, min normal exponent, max exponent)
F16 = (11, -14, 15)
F32 = (24, -126, 127)


def round_binary(x: Fraction, mant: int, emin: int, emax: int):
    """Round a rational to the nearest binary float (ties to even significand).

    Returns a Fraction, or +-math.inf on overflow.  Subnormals use emin's spacing.
    """
    x = Fraction(x)
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    ulp = Fraction(2) ** (e - (mant - 1))
    m = a / ulp
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * ulp
    maxf = (2 - Fraction(2) ** (1 - mant)) * Fraction(2) ** emax
    if r > maxf:
        return sign * math.inf
    return sign * r


def fr(v) -> Fraction:
    """Exact rational value of a finite float (numpy or Python)."""
    return Fraction(float(v))

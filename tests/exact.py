"""Exact rational arithmetic with explicit IEEE rounding, for brute-force pins.

Everything here works on ``fractions.Fraction`` and rounds to binary32 /
binary16 by construction (round to nearest, ties to even), so a pin built on
it does not depend on numpy's or the compiler's floating-point arithmetic.
"""
from __future__ import annotations

import math
from fractions import Fraction


def _round_to_format(x: Fraction, mant_bits: int, emin: int) -> Fraction:
    """Round x to the nearest number with ``mant_bits`` significand bits
    (including the implicit one) and minimum normal exponent ``emin``;
    subnormals are handled; overflow is not (callers stay in range)."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    # exponent e with 2**e <= a < 2**(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    ulp = Fraction(2) ** (e - (mant_bits - 1))
    m = a / ulp
    n = math.floor(m)
    r = m - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * ulp


def f32(x) -> Fraction:
    """Round to IEEE binary32."""
    return _round_to_format(Fraction(x), 24, -126)


def f16(x) -> Fraction:
    """Round to IEEE binary16."""
    return _round_to_format(Fraction(x), 11, -14)


def fr(x) -> Fraction:
    """Exact rational value of a Python / numpy float."""
    return Fraction(float(x))


def round_half_away(x: Fraction) -> int:
    n = math.floor(abs(x) + Fraction(1, 2))
    return n if x >= 0 else -n


def round_half_even(x: Fraction) -> int:
    n = math.floor(x)
    r = x - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return n

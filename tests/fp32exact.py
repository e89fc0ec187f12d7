"""Exact IEEE-754 binary32 arithmetic on rationals, for pinning the oracle.

``round_f32`` rounds an exact rational to the nearest binary32 value (ties to
even, gradual underflow); ``fma_f32`` is one fused multiply-add with a single
rounding. Used on tiny inputs only (pure Python, slow).
"""

from fractions import Fraction

import numpy as np


def round_f32(q: Fraction) -> Fraction:
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = -q if q < 0 else q
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    quantum = Fraction(2) ** (e - 23)
    m = a / quantum
    n = m.numerator // m.denominator
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * quantum


def fma_f32(a, b, c) -> Fraction:
    return round_f32(Fraction(a) * Fraction(b) + Fraction(c))


def add_f32(a, b) -> Fraction:
    return round_f32(Fraction(a) + Fraction(b))


def to_f32(q: Fraction) -> np.float32:
    v = np.float32(float(q))
    assert Fraction(float(v)) == q, "value not representable in binary32"
    return v

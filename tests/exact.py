"""Exact-rational helpers for the oracle's pins (test side only).

Independent of the oracle: fp32 rounding is done here from its definition
(round to nearest, ties to even, 24-bit significand) on Python Fractions, not
by any float32 hardware operation.
"""

from fractions import Fraction

import numpy as np


def f32_round(q: Fraction) -> Fraction:
    """Round a non-negative rational to the nearest fp32 value, ties to even.

    Only the normal range is needed here (no subnormals, no overflow).
    """
    q = Fraction(q)
    if q < 0:
        return -f32_round(-q)
    if q == 0:
        return Fraction(0)
    e = q.numerator.bit_length() - q.denominator.bit_length()
    # settle e so that 2^e <= q < 2^(e+1)
    while Fraction(2) ** e > q:
        e -= 1
    while Fraction(2) ** (e + 1) <= q:
        e += 1
    unit = Fraction(2) ** (e - 23)          # ulp of the binade
    m = q / unit                            # in [2^23, 2^24)
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return fl * unit


def as_fraction(x) -> Fraction:
    """Exact value of a float32/float64 number."""
    return Fraction(float(x))


def symmetric_pad(plane: np.ndarray, pad_lo: int, pad_hi: int) -> np.ndarray:
    """Half-sample symmetric extension by numpy's own definition of "symmetric"."""
    return np.pad(plane, ((pad_lo, pad_hi), (pad_lo, pad_hi)), mode="symmetric")

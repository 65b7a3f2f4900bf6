"""Exact brute-force MXFP4 reference in rational arithmetic (for pinning the oracle).

Independent of the oracle's code: the block exponent is found by searching
powers of two with exact Fraction comparisons, and every element is rounded
by scanning all eight e2m1 magnitudes for the nearest one, an exact tie going
to the magnitude whose code is even (mantissa bit 0).
"""

import math
from fractions import Fraction

MAGS = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2),
        Fraction(2), Fraction(3), Fraction(4), Fraction(6)]


def floor_log2_exact(v: Fraction) -> int:
    """floor(log2(v)) for v > 0: start from the integer bit lengths of the
    numerator and denominator, then correct with exact comparisons."""
    e = v.numerator.bit_length() - v.denominator.bit_length()
    while Fraction(2) ** e > v:
        e -= 1
    while Fraction(2) ** (e + 1) <= v:
        e += 1
    return e


def encode_block(xs, only=None):
    """xs: 32 Python floats. Returns (scale_code, [unpacked codes]).

    With only=n, the scale still comes from all 32 values but only the first
    n elements are encoded (the rest of such test blocks is zero padding)."""
    amax = Fraction(max(abs(x) for x in xs))        # abs/max of floats are exact
    if only is not None:
        xs = xs[:only]
    fr = [Fraction(x) for x in xs]
    if amax == 0:
        shared = -127
    else:
        shared = max(-127, min(127, floor_log2_exact(amax) - 2))
    scale = Fraction(2) ** shared
    codes = []
    for x, v in zip(xs, fr):
        q = abs(v) / scale
        best, best_d = None, None
        for c, mag in enumerate(MAGS):
            d = abs(q - mag)
            if best is None or d < best_d or (d == best_d and c % 2 == 0):
                best, best_d = c, d
        sign = 1 if math.copysign(1.0, x) < 0 else 0
        codes.append(sign << 3 | best)
    return shared + 127, codes


def dot_exact(a_vals, b_vals):
    """Exact sum of products of two equal-length sequences of Fractions."""
    return sum((x * y for x, y in zip(a_vals, b_vals)), Fraction(0))

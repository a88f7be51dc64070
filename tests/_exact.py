"""Exact-rational helpers for pinning the oracle (CPU only, no numpy rounding).

Everything here works on fractions.Fraction so that rounding happens only
where a function says so, by the IEEE round-to-nearest-even rule applied to
the exact rational value.
"""
from __future__ import annotations

from fractions import Fraction

FMT = {"f16": (10, -14, 15), "bf16": (7, -126, 127), "f32": (23, -126, 127)}


def round_half_even(x: Fraction) -> int:
    f = x.numerator // x.denominator          # floor
    r = x - f
    if r > Fraction(1, 2):
        return f + 1
    if r < Fraction(1, 2):
        return f
    return f if f % 2 == 0 else f + 1


def exact_round(x: Fraction, fmt: str) -> Fraction:
    """Round a rational to the nearest value of a binary format (ties to even)."""
    mant, emin, emax = FMT[fmt]
    if x == 0:
        return Fraction(0)
    sgn = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # fix e so that 2^e <= a < 2^(e+1)
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    step = Fraction(2) ** (e - mant)
    q = round_half_even(a / step) * step
    maxfin = (2 - Fraction(1, 2 ** mant)) * Fraction(2) ** emax
    if q > maxfin:
        raise OverflowError
    return sgn * q


def fl32(x: Fraction) -> Fraction:
    return exact_round(x, "f32")

"""Floating-point storage formats for the CPU oracle (test infrastructure).

Every value the oracle handles is kept in float64 (or as an exact integer);
rounding to a storage format happens only where the layer's definition rounds.

* ``round_to_format`` rounds float64 values to the nearest value of a binary
  floating-point format with round-half-to-even, subnormals and overflow to
  infinity: the textbook IEEE 754 rule written out with frexp/ldexp/rint.
* fp16 conversion uses numpy's IEEE half conversion; fp32 numpy's float32.
* bf16 values are uint16 bit patterns; widening to fp32 is the exact 16-bit
  shift, narrowing is ``round_to_format`` with 7 fraction bits and the fp32
  exponent range.

Pinned by tests/test_oracle_formats.py against numpy's float16/float32
conversions and torch's bfloat16 conversion (independent implementations).
"""
from __future__ import annotations

import numpy as np

# (fraction bits, minimum normal exponent, maximum exponent)
FMT = {
    "f16": (10, -14, 15),
    "bf16": (7, -126, 127),
    "f32": (23, -126, 127),
}


def round_to_format(x, fmt: str) -> np.ndarray:
    """Round float64 values to nearest-even in format ``fmt``; returns float64."""
    mant, emin, emax = FMT[fmt]
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                       # |x| in [2^(e-1), 2^e)
    lead = np.maximum(e - 1, emin)           # exponent of the leading bit (subnormals: emin)
    q = np.rint(np.ldexp(x, mant - lead))    # exact power-of-two scaling, then half-even
    r = np.ldexp(q, lead - mant)
    maxfin = np.ldexp(2.0 - 2.0 ** -mant, emax)
    big = np.abs(r) > maxfin
    if np.any(big):
        r = np.where(big, np.copysign(np.inf, x), r)
    nan = np.isnan(x)
    if np.any(nan):
        r = np.where(nan, np.nan, r)
    return r


def bf16_bits_to_f64(u16) -> np.ndarray:
    u = np.asarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x) -> np.ndarray:
    r = round_to_format(x, "bf16").astype(np.float32)   # exact: bf16 values are fp32 values
    return (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def to_f64(x, dt: str) -> np.ndarray:
    """Exact float64 value of a stored tensor."""
    if dt == "bf16":
        return bf16_bits_to_f64(x)
    if dt in ("f16", "f32"):
        return np.asarray(x).astype(np.float64)
    raise ValueError(dt)


def from_f64(y, dt: str) -> np.ndarray:
    """One round-to-nearest-even of float64 values into storage dtype ``dt``."""
    y = np.asarray(y, dtype=np.float64)
    if dt == "f32":
        return y.astype(np.float32)
    if dt == "f16":
        return y.astype(np.float16)
    if dt == "bf16":
        return f64_to_bf16_bits(y)
    raise ValueError(dt)


def to_half(x, dt: str) -> np.ndarray:
    """Cast a stored tensor to fp16 with round-to-nearest-even (exact for fp16)."""
    if dt == "f16":
        return np.asarray(x, dtype=np.float16)
    if dt == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float16)
    if dt == "bf16":
        return bf16_bits_to_f64(x).astype(np.float32).astype(np.float16)
    raise ValueError(dt)


def ulp(y, dt: str) -> np.ndarray:
    """Spacing of format ``dt`` at the magnitude of y (float64)."""
    mant, emin, _ = FMT[dt]
    y = np.asarray(y, dtype=np.float64)
    _, e = np.frexp(y)
    lead = np.where(y == 0, emin, np.maximum(e - 1, emin))
    return np.ldexp(1.0, lead - mant)

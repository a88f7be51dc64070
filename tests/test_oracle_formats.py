"""Pins of the oracle's storage-format conversions (CPU).

round_to_format is checked against independent implementations: numpy's
float16 and float32 conversions and torch's bfloat16 conversion, on random
values, exact ties, subnormals and overflow; and against exact rational
rounding on a sample.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

from oracle.formats import (bf16_bits_to_f64, f64_to_bf16_bits, from_f64, round_to_format, to_half,
                            ulp)
from tests._exact import exact_round


def _wide_f64(n, seed):
    g = np.random.default_rng(seed)
    mant = g.uniform(-1.0, 1.0, n)
    ex = g.integers(-30, 20, n)
    return np.ldexp(mant, ex)


def _ties(fmt_dtype, n, seed):
    """Exact midpoints between consecutive values of a numpy float format."""
    g = np.random.default_rng(seed)
    if fmt_dtype == np.float16:
        bits = g.integers(0, 0x7BFF, n).astype(np.uint16)
        a = bits.view(np.float16).astype(np.float64)
        b = (bits + 1).view(np.float16).astype(np.float64)
    else:
        bits = g.integers(0, 0x7F7FFFFF, n).astype(np.uint32)
        a = bits.view(np.float32).astype(np.float64)
        b = (bits + 1).view(np.float32).astype(np.float64)
    mid = (a + b) / 2.0
    sign = np.where(g.random(n) < 0.5, -1.0, 1.0)
    return mid * sign


def test_f16_matches_numpy_random_and_ties():
    x = np.concatenate([_wide_f64(200000, 1), _ties(np.float16, 50000, 2),
                        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e6, -1e6,
                                  2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -26])])
    mine = round_to_format(x, "f16")
    ref = x.astype(np.float16).astype(np.float64)
    assert np.array_equal(mine, ref)
    assert np.array_equal(np.signbit(mine), np.signbit(ref))


def test_f32_matches_numpy_random_and_ties():
    x = np.concatenate([np.ldexp(np.random.default_rng(3).uniform(-1, 1, 200000),
                                 np.random.default_rng(4).integers(-150, 128, 200000)),
                        _ties(np.float32, 50000, 5)])
    mine = round_to_format(x, "f32")
    with np.errstate(over="ignore"):
        ref = x.astype(np.float32).astype(np.float64)
    assert np.array_equal(mine, ref)


def test_bf16_matches_torch_on_fp32_inputs():
    g = np.random.default_rng(6)
    bits = g.integers(0, 2 ** 32, 1_000_000, dtype=np.uint64).astype(np.uint32)
    x32 = bits.view(np.float32)
    x32 = x32[np.isfinite(x32)]
    # add exact bf16 midpoints
    hb = g.integers(0, 0x7F7F, 20000).astype(np.uint32)
    mids = ((hb << 16) | 0x8000).view(np.float32)
    x32 = np.concatenate([x32, mids, -mids])
    ref = torch.from_numpy(x32.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    mine = f64_to_bf16_bits(x32.astype(np.float64))
    assert np.array_equal(mine, ref)


def test_bf16_widening_exhaustive():
    u = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    mine = bf16_bits_to_f64(u)
    ref = torch.from_numpy(u.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    same = (mine == ref) | (np.isnan(mine) & np.isnan(ref))
    assert same.all()


def test_bf16_to_half_exhaustive():
    u = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = bf16_bits_to_f64(u)
    fin = np.isfinite(v)
    mine = to_half(u[fin], "bf16").astype(np.float64)
    ref = round_to_format(v[fin], "f16")
    assert np.array_equal(mine, ref)


def test_from_f64_half_is_single_rounding():
    # numpy's float64 -> float16 conversion must round once (no detour via fp32)
    x = np.concatenate([_wide_f64(200000, 7), _ties(np.float16, 20000, 8)])
    # nudge ties by far less than an fp32 ulp: single rounding must see the nudge
    x = np.concatenate([x, np.nextafter(_ties(np.float16, 20000, 9), np.inf)])
    assert np.array_equal(from_f64(x, "f16").astype(np.float64), round_to_format(x, "f16"))


def test_round_to_format_vs_exact_rationals():
    g = np.random.default_rng(10)
    x = _wide_f64(3000, 11)
    for fmt in ("f16", "bf16", "f32"):
        r = round_to_format(x, fmt)
        for xi, ri in zip(x, r):
            if not np.isfinite(ri):
                with pytest.raises(OverflowError):
                    exact_round(Fraction(float(xi)), fmt)
                continue
            assert Fraction(float(ri)) == exact_round(Fraction(float(xi)), fmt), (fmt, xi)
    del g


def test_ulp():
    assert ulp(np.array([1.0]), "f16")[0] == 2.0 ** -10
    assert ulp(np.array([1.0]), "bf16")[0] == 2.0 ** -7
    assert ulp(np.array([0.0]), "f16")[0] == 2.0 ** -24

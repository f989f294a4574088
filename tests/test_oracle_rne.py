"""Pins of the oracle's 16-bit conversions against the IEEE 754 definition.

Round to nearest, ties to even, is fixed by three facts checked here for every
pair of neighbouring patterns: exact values map to themselves, anything below
the midpoint maps down and above it maps up, and the exact midpoint maps to
the pattern with an even last bit.  Overflow to infinity and the sign of zero
follow the same rule.
"""
import numpy as np
import pytest

from oracle import BF16, F16, rne16, widen


@pytest.mark.parametrize("dtype,max_finite", [(F16, 0x7BFF), (BF16, 0x7F7F)])
def test_exact_values_round_to_themselves(dtype, max_finite):
    pats = np.arange(0, max_finite + 1, dtype=np.uint32).astype(np.uint16)
    for sign in (0, 0x8000):
        p = pats | np.uint16(sign)
        assert np.array_equal(rne16(widen(p, dtype), dtype), p)


@pytest.mark.parametrize("dtype,max_finite", [(F16, 0x7BFF), (BF16, 0x7F7F)])
def test_midpoints_and_neighbours(dtype, max_finite):
    lo = np.arange(0, max_finite, dtype=np.uint32).astype(np.uint16)
    hi = (lo.astype(np.uint32) + 1).astype(np.uint16)
    vlo, vhi = widen(lo, dtype), widen(hi, dtype)
    mid = (vlo + vhi) / 2            # exact in fp64: at most 12 significant bits
    assert np.all((mid > vlo) & (mid < vhi))
    even = np.where(lo % 2 == 0, lo, hi)
    assert np.array_equal(rne16(mid, dtype), even)
    assert np.array_equal(rne16(np.nextafter(mid, -np.inf), dtype), lo)
    assert np.array_equal(rne16(np.nextafter(mid, np.inf), dtype), hi)
    assert np.array_equal(rne16(-mid, dtype), even | np.uint16(0x8000))


def test_known_patterns():
    # fp16: 1.0 = 0x3C00, max 65504 = 0x7BFF, smallest subnormal 2^-24 = 0x0001
    assert rne16(np.array([1.0, 65504.0, 2.0 ** -24, -2.0]), F16).tolist() == [0x3C00, 0x7BFF, 0x0001, 0xC000]
    # bf16: 1.0 = 0x3F80, smallest subnormal 2^-133 = 0x0001, 3.0 = 0x4040
    assert rne16(np.array([1.0, 2.0 ** -133, 3.0, -0.5]), BF16).tolist() == [0x3F80, 0x0001, 0x4040, 0xBF00]
    # widening: the decode of a few patterns by their format definition
    assert widen(np.array([0x3F80, 0x4049, 0x0001], np.uint16), BF16).tolist() == [1.0, 3.140625, 2.0 ** -133]
    assert widen(np.array([0x3555, 0x0001], np.uint16), F16).tolist() == [0.333251953125, 2.0 ** -24]


def test_overflow_and_specials():
    # fp16: the midpoint between 65504 and 65536 is 65520; the tie goes to the even pattern, infinity
    assert rne16(np.array([65519.99, 65520.0, 1e6, -1e6, np.inf]), F16).tolist() == \
        [0x7BFF, 0x7C00, 0x7C00, 0xFC00, 0x7C00]
    big = (2 - 2 ** -7) * 2.0 ** 127
    assert rne16(np.array([big, big + 2.0 ** 119, np.nan]), BF16).tolist() == [0x7F7F, 0x7F80, 0x7FC0]
    assert rne16(np.array([0.0, -0.0, -1e-300]), F16).tolist() == [0x0000, 0x8000, 0x8000]


def test_f16_matches_numpy_direct_conversion():
    # numpy converts float64 -> float16 directly with round-to-nearest-even
    g = np.random.default_rng(7)
    a = np.concatenate([g.standard_normal(200_000) * s for s in (1e-7, 1e-5, 0.02, 1.0, 300.0, 6e4)])
    assert np.array_equal(rne16(a, F16), a.astype(np.float16).view(np.uint16))

"""Pins for oracle/rounding.py: exact rational rounding, torch's float32 -> bf16
conversion, numpy's float32 cast."""

import math
from fractions import Fraction

import numpy as np
import torch

from oracle.rounding import bf16_bits, round_bf16, round_f32


def _rne_fraction(x: float, mant_bits: int, min_exp: int) -> float:
    """Round x to `mant_bits` significant bits, ties to even, exactly."""
    if x == 0.0:
        return 0.0
    fx = Fraction(x)
    e = math.frexp(x)[1]
    e = max(e, min_exp)
    q = Fraction(2) ** (e - mant_bits)
    n = fx / q
    fl = math.floor(n)
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return float(fl * q)


def test_bf16_matches_exact_rounding_random():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(4000) * np.exp2(rng.integers(-30, 30, size=4000))
    got = round_bf16(x)
    want = np.array([_rne_fraction(float(v), 8, -125) for v in x])
    assert np.array_equal(got, want)


def test_bf16_ties_go_to_even():
    rng = np.random.default_rng(1)
    for _ in range(500):
        # a bf16 value m * 2**k with 8-bit m, plus exactly half an ulp
        m = int(rng.integers(128, 256))
        k = int(rng.integers(-20, 20))
        x = (m + 0.5) * 2.0 ** k
        want = (m + (m % 2)) * 2.0 ** k
        assert round_bf16(x) == want
        assert round_bf16(-x) == -want
        # just above / below the tie
        up = math.nextafter(x, math.inf)
        dn = math.nextafter(x, -math.inf)
        assert round_bf16(up) == (m + 1) * 2.0 ** k
        assert round_bf16(dn) == m * 2.0 ** k


def test_bf16_matches_torch_for_float32_inputs():
    x = np.random.default_rng(2).standard_normal(100_000).astype(np.float32) * 3
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(round_bf16(x.astype(np.float64)), want)


def test_double_rounding_is_avoided():
    """A float64 just above a bf16 tie must round up, even though rounding it
    to float32 first would land exactly on the tie and round to even."""
    m, k = 130, 0                   # even 8-bit mantissa: an exact tie stays at m
    tie = (m + 0.5) * 2.0 ** k
    x = tie + 2.0 ** (k - 30)       # above the tie by less than a float32 ulp
    assert np.float32(x) == np.float32(tie)
    assert round_bf16(x) == (m + 1) * 2.0 ** k


def test_f32_matches_exact_rounding():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(2000) * np.exp2(rng.integers(-20, 20, size=2000))
    want = np.array([_rne_fraction(float(v), 24, -125) for v in x])
    assert np.array_equal(round_f32(x), want)


def test_bits_roundtrip():
    v = round_bf16(np.random.default_rng(4).standard_normal(1000))
    bits = bf16_bits(v)
    back = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(back, v)

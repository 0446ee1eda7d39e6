"""Pins for oracle/quant.py (int8 rows with one absmax scale per row)."""

import numpy as np
import pytest

from oracle.quant import dequantize_rows, quantize_dequantize, quantize_rows


def test_exact_multiples_round_trip():
    rng = np.random.default_rng(1)
    for e in (-9, -3, 0, 4):
        codes = rng.integers(-127, 128, size=(20, 128))
        codes[:, 5] = 127 * np.where(rng.random(20) < 0.5, 1, -1)  # largest |code| is 127
        x = codes.astype(np.float64) * 2.0 ** e
        q, s = quantize_rows(x)
        assert np.array_equal(q, codes.astype(np.int8))
        assert np.all(s == np.float32(2.0 ** e))
        assert np.array_equal(dequantize_rows(q, s), x)


def test_error_bound_and_extremes():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((500, 64)) * rng.uniform(1e-3, 10, size=(500, 1))
    q, s = quantize_rows(x)
    err = np.abs(dequantize_rows(q, s) - x)
    # half a step, plus the float32 rounding of the scale over 127 steps
    assert np.all(err <= s[:, None] * (0.5 + 127 * 2.0 ** -24) + 1e-300)
    am = np.abs(x).argmax(axis=1)
    assert np.all(np.abs(q[np.arange(500), am]) == 127)
    assert np.all(np.abs(q.astype(np.int32)) <= 127)


def test_symmetry_and_zero():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((50, 128))
    q1, s1 = quantize_rows(x)
    q2, s2 = quantize_rows(-x)
    assert np.array_equal(q1, -q2) and np.array_equal(s1, s2)
    q, s = quantize_rows(np.zeros((3, 128)))
    assert np.all(s == 0) and np.all(q == 0)
    assert np.all(quantize_dequantize(np.zeros((3, 128))) == 0)


def test_nearest_code_brute_force():
    """The code of every element is the integer in [-127, 127] nearest to
    x / s (ties to the even one), found by trying all 255."""
    rng = np.random.default_rng(4)
    x = rng.standard_normal((40, 16))
    x[0, :4] = [1.0, 0.5 / 127 * 3, -2.5 / 127, 0.0]  # includes exact ties x / s = k + 1/2
    q, s = quantize_rows(x)
    cands = np.arange(-127, 128, dtype=np.float64)
    for r in range(x.shape[0]):
        s64 = float(s[r])
        for i in range(x.shape[1]):
            d = np.abs(x[r, i] / s64 - cands)
            best = cands[d == d.min()]
            want = best[0] if best.size == 1 else best[best % 2 == 0][0]
            assert q[r, i] == want, (r, i)


@pytest.mark.parametrize("d", [64, 128])
def test_relative_error_of_gaussian_rows(d):
    """For N(0, 1) rows the dequantised row is within ~1% of the row in norm
    (step = absmax / 127; the page's 'controllable loss of precision')."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((200, d))
    rel = np.linalg.norm(quantize_dequantize(x) - x, axis=1) / np.linalg.norm(x, axis=1)
    assert rel.max() < 0.02

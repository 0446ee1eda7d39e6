"""Pins for oracle/rope.py: what any rotary embedding must satisfy.  The
pairings and frequencies themselves are pinned against library
implementations in tests/test_oracle_rope_library.py."""

import math

import numpy as np
import pytest

from oracle.rope import inv_freq, rope

STYLES = ["interleaved", "half"]


@pytest.mark.parametrize("style", STYLES)
def test_position_zero_is_identity(style):
    x = np.random.default_rng(0).standard_normal((5, 3, 64))
    assert np.array_equal(rope(x, 0, 10000.0, style), x)


@pytest.mark.parametrize("style", STYLES)
def test_norm_preserved(style):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((50, 128))
    pos = rng.integers(0, 300_000, size=50)
    y = rope(x, pos, 10000.0, style)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)


@pytest.mark.parametrize("style", STYLES)
@pytest.mark.parametrize("pos", [0, 1, 2, 7, 1000, 262_144])
def test_d2_rotates_by_position_radians(style, pos):
    """With one pair, theta_0 = 1: the unit vector goes to (cos pos, sin pos)."""
    y = rope(np.array([1.0, 0.0]), pos, 10000.0, style)
    assert np.allclose(y, [math.cos(pos), math.sin(pos)], atol=1e-12)
    y = rope(np.array([0.0, 1.0]), pos, 10000.0, style)
    assert np.allclose(y, [-math.sin(pos), math.cos(pos)], atol=1e-12)


@pytest.mark.parametrize("style", STYLES)
def test_scores_depend_only_on_position_difference(style):
    """Relative-position property: <R(q,t), R(k,p)> is unchanged when both
    positions shift by the same amount."""
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal(128), rng.standard_normal((20, 128))
    t, p = 5000, rng.integers(0, 5000, size=20)
    base = rope(k, p, 10000.0, style) @ rope(q, t, 10000.0, style)
    for shift in (1, 1000, 250_000):
        moved = rope(k, p + shift, 10000.0, style) @ rope(q, t + shift, 10000.0, style)
        assert np.allclose(moved, base, rtol=1e-9, atol=1e-9)


@pytest.mark.parametrize("style", STYLES)
def test_rotations_compose(style):
    x = np.random.default_rng(3).standard_normal((4, 64))
    assert np.allclose(rope(rope(x, 300, 500.0, style), 45, 500.0, style),
                       rope(x, 345, 500.0, style), atol=1e-12)


def test_styles_are_the_same_map_up_to_a_coordinate_permutation():
    d = 16
    perm = np.array([2 * i for i in range(d // 2)] + [2 * i + 1 for i in range(d // 2)])
    x = np.random.default_rng(4).standard_normal((3, d))
    inter = rope(x, [5, 99, 1234], 10000.0, "interleaved")
    half = rope(x[:, perm], [5, 99, 1234], 10000.0, "half")
    assert np.allclose(half, inter[:, perm], atol=1e-12)


def test_frequencies_decrease_from_one():
    th = inv_freq(128, 10000.0)
    assert th[0] == 1.0 and np.all(np.diff(th) < 0) and th[-1] > 1.0 / 10000.0


def test_pins_catch_planted_mistakes():
    x = np.array([1.0, 0.0])

    def wrong_sign(v, pos):  # rotation by -pos
        c, s = math.cos(pos), math.sin(pos)
        return np.array([v[0] * c + v[1] * s, -v[0] * s + v[1] * c])

    def not_a_rotation(v, pos):  # sign slip in one term
        c, s = math.cos(pos), math.sin(pos)
        return np.array([v[0] * c + v[1] * s, v[0] * s + v[1] * c])

    assert not np.allclose(wrong_sign(x, 3), [math.cos(3), math.sin(3)])
    y = not_a_rotation(np.array([0.6, 0.8]), 1.0)
    assert not math.isclose(np.linalg.norm(y), 1.0)

"""Pins for the cache-position-shifting reading ([sink]: positions inside
the attention are the keys' indices in the cache, sinks then window)."""

import numpy as np
import pytest

from oracle.attention import attend_heads
from oracle.decode import ring_cache_positions, ring_shifted_expected
from oracle.ring import concat_prune, resident_positions
from oracle.rope import rope
from synth import TENSOR_K, TENSOR_Q, TENSOR_V, RingWorkload


@pytest.mark.parametrize("sinks,window", [(4, 16), (1, 2), (0, 4), (4, 4), (2, 9)])
def test_cache_positions_are_the_managers_indices(sinks, window):
    """The [sink] cache manager keeps a list (sinks, then the recent window)
    in order: a key's cache position is its index in that list."""
    for t in range(0, 5 * (sinks + window)):
        lst = concat_prune([[p] for p in range(t + 1)], sinks, window)
        assert ring_cache_positions(t, sinks, window) == {p: i for i, p in enumerate(lst)}


def _w(**kw):
    base = dict(name="s", seed=91, batch=1, num_q_heads=4, num_kv_heads=2, head_dim=16,
                dtype="f32", window=12, sinks=3, rope_base=100.0, scale=1.0, decode_steps=40,
                history="prefill:1")
    base.update(kw)
    return RingWorkload(**base)


def _absolute(w, b, step):
    """Attention with absolute positions, unrounded."""
    t = int(w.decode_positions(step)[b])
    pos = np.asarray(resident_positions(t, w.sinks, w.window), dtype=np.int64)
    k = rope(w.rows(TENSOR_K, b, pos), pos[:, None], w.rope_base)
    q = rope(w.rows(TENSOR_Q, b, [t])[0], t, w.rope_base)
    return attend_heads(q, k, w.rows(TENSOR_V, b, pos).astype(np.float64))


def test_below_capacity_equals_absolute():
    """Before anything is evicted the cache index is the position itself."""
    w = _w()
    for step in range(0, w.sinks + w.window - 1):
        a, _ = _absolute(w, 0, step)
        s, _ = ring_shifted_expected(w, 0, step)
        assert np.abs(a - s).max() < 1e-12


def test_no_sinks_equals_absolute():
    """Without sinks the cache is one contiguous run of positions: every
    distance to the query is unchanged, and so is the output (RoPE scores
    depend on distances only)."""
    w = _w(sinks=0)
    for step in range(0, 40, 3):
        a, _ = _absolute(w, 0, step)
        s, _ = ring_shifted_expected(w, 0, step)
        assert np.abs(a - s).max() < 1e-10


def test_shifting_changes_only_the_sinks():
    """Past capacity the window keys keep their distance to the query and the
    sinks move to distance S + W - 1 - s: with V zero on the window rows the
    outputs differ, with the sinks' V zero and their keys zero (no sink
    weight depends on a rotation then) they agree."""
    w = _w()
    step = 35  # t = 35 > S + W - 1 = 14
    t = int(w.decode_positions(step)[0])
    pos = np.asarray(resident_positions(t, w.sinks, w.window), dtype=np.int64)
    cpos = ring_cache_positions(t, w.sinks, w.window)
    c = np.asarray([cpos[p] for p in pos])
    k_raw = w.rows(TENSOR_K, 0, pos).astype(np.float64)
    v = w.rows(TENSOR_V, 0, pos).astype(np.float64)
    q_raw = w.rows(TENSOR_Q, 0, [t])[0]
    sink = pos < w.sinks
    k0 = k_raw.copy()
    k0[sink] = 0.0
    v0 = v.copy()
    v0[sink] = 0.0
    a, _ = attend_heads(rope(q_raw, t, w.rope_base), rope(k0, pos[:, None], w.rope_base), v0)
    s, _ = attend_heads(rope(q_raw, cpos[t], w.rope_base), rope(k0, c[:, None], w.rope_base), v0)
    assert np.abs(a - s).max() < 1e-12
    a, _ = _absolute(w, 0, step)
    s, _ = ring_shifted_expected(w, 0, step)
    assert np.abs(a - s).max() > 1e-6

"""Pins for oracle/attention.py and oracle/decode.py: torch's float64
scaled_dot_product_attention, scipy's logsumexp, a pure-Python double loop,
closed forms (V = 1, K = 0), masked-full = windowed."""

import math

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

from oracle.attention import attend, attend_heads, attend_loops, attend_masked
from oracle.decode import ring_expected, ring_query, ring_rows, ring_slot_table
from oracle.ring import resident_positions, slot_contents
from synth import RingWorkload


def _sdpa(q, K, V, scale=None):
    qt = torch.from_numpy(np.asarray(q, np.float64))[None, None, None, :]
    kt = torch.from_numpy(np.asarray(K, np.float64))[None, None]
    vt = torch.from_numpy(np.asarray(V, np.float64))[None, None]
    return F.scaled_dot_product_attention(qt, kt, vt, scale=scale)[0, 0, 0].numpy()


def test_matches_torch_sdpa():
    rng = np.random.default_rng(0)
    for n, d in [(1, 8), (7, 64), (300, 128), (4100, 128)]:
        q, K, V = rng.standard_normal(d), rng.standard_normal((n, d)), rng.standard_normal((n, d))
        o, lse = attend(q, K, V)
        assert np.allclose(o, _sdpa(q, K, V), rtol=1e-12, atol=1e-13)
        assert math.isclose(lse, scipy.special.logsumexp(K @ q / math.sqrt(d)), rel_tol=1e-13)
        o2, _ = attend(q, K, V, scale=0.3)
        assert np.allclose(o2, _sdpa(q, K, V, scale=0.3), rtol=1e-12, atol=1e-13)


def test_gqa_grouping_matches_torch():
    """Query head h reads kv head h // g (torch's enable_gqa uses the same rule)."""
    rng = np.random.default_rng(1)
    hq, hkv, n, d = 24, 4, 50, 32
    q = rng.standard_normal((hq, d))
    K, V = rng.standard_normal((n, hkv, d)), rng.standard_normal((n, hkv, d))
    o, _ = attend_heads(q, K, V)
    qt = torch.from_numpy(q)[None, :, None, :]
    kt = torch.from_numpy(K.transpose(1, 0, 2).copy())[None]
    vt = torch.from_numpy(V.transpose(1, 0, 2).copy())[None]
    want = F.scaled_dot_product_attention(qt, kt, vt, enable_gqa=True)[0, :, 0, :].numpy()
    assert np.allclose(o, want, rtol=1e-12, atol=1e-13)


def test_loops_equal_vectorised_on_tiny_shapes():
    rng = np.random.default_rng(2)
    for n, d in [(1, 2), (2, 2), (3, 4), (6, 2)]:
        q, K, V = rng.standard_normal(d), rng.standard_normal((n, d)), rng.standard_normal((n, d))
        o1, l1 = attend(q, K, V)
        o2, l2 = attend_loops(q.tolist(), K.tolist(), V.tolist())
        assert np.allclose(o1, o2, rtol=1e-13, atol=1e-14)
        assert math.isclose(l1, l2, rel_tol=1e-13)


def test_weights_sum_to_one():
    """[sink]: the weights sum to one, so V = 1 gives output 1 exactly-ish."""
    rng = np.random.default_rng(3)
    q, K = rng.standard_normal(64) * 4, rng.standard_normal((1000, 64)) * 4
    o, _ = attend(q, K, np.ones((1000, 64)))
    assert np.allclose(o, 1.0, atol=1e-14)


def test_zero_keys_give_the_mean_of_values():
    rng = np.random.default_rng(4)
    V = rng.standard_normal((333, 16))
    o, lse = attend(rng.standard_normal(16), np.zeros((333, 16)), V)
    assert np.allclose(o, V.mean(axis=0), atol=1e-14)
    assert math.isclose(lse, math.log(333), rel_tol=1e-14)


def test_empty_set():
    o, lse = attend(np.ones(8), np.zeros((0, 8)), np.zeros((0, 8)))
    assert np.array_equal(o, np.zeros(8)) and lse == -math.inf


@pytest.mark.parametrize("sinks,window", [(4, 16), (0, 8), (2, 5)])
def test_masked_full_history_equals_windowed_set(sinks, window):
    """[ring] §3.1 / [pool] mask: masking everything outside R(t) with -inf over
    the full history gives the same result as attending R(t) alone."""
    rng = np.random.default_rng(5)
    d = 32
    for t in (0, 3, window, sinks + window + 7, 200):
        K, V = rng.standard_normal((t + 1, d)), rng.standard_normal((t + 1, d))
        q = rng.standard_normal(d)
        r = resident_positions(t, sinks, window)
        keep = np.zeros(t + 1, bool)
        keep[r] = True
        o1, l1 = attend_masked(q, K, V, keep)
        o2, l2 = attend(q, K[r], V[r])
        assert np.allclose(o1, o2, rtol=1e-14, atol=1e-15)
        assert math.isclose(l1, l2, rel_tol=1e-14)


def _tiny(dtype="f32", **kw):
    base = dict(name="t", seed=11, batch=2, num_q_heads=4, num_kv_heads=2, head_dim=16,
                dtype=dtype, window=8, sinks=2, rope_base=10000.0, scale=1.0,
                decode_steps=30, history="prefill:3")
    base.update(kw)
    return RingWorkload(**base)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ring_decode_below_capacity_is_full_causal_attention(dtype):
    """While t + 1 <= S + W nothing is evicted ([sink] manager keeps all below
    capacity): the decode output is plain causal attention over 0..t."""
    w = _tiny(dtype)
    for step in range(0, w.slots - 3):
        t = int(w.decode_positions(step)[1])
        assert t + 1 <= w.slots
        out, lse = ring_expected(w, 1, step)
        k, v = ring_rows(w, 1, range(t + 1))
        q = ring_query(w, 1, t)
        for h in range(w.num_q_heads):
            kv = h // w.group
            want = _sdpa(q[h], k[:, kv], v[:, kv])
            assert np.allclose(out[h], want, rtol=1e-12, atol=1e-13)


def test_ring_decode_uses_only_the_resident_set():
    w = _tiny("f32")
    step = 25
    t = int(w.decode_positions(step)[0])
    out, _ = ring_expected(w, 0, step)
    full_k, full_v = ring_rows(w, 0, range(t + 1))
    keep = np.zeros(t + 1, bool)
    keep[resident_positions(t, w.sinks, w.window)] = True
    q = ring_query(w, 0, t)
    for h in range(w.num_q_heads):
        o, _ = attend_masked(q[h], full_k[:, h // w.group], full_v[:, h // w.group], keep)
        assert np.allclose(out[h], o, rtol=1e-13, atol=1e-14)
    # and it differs from attending the whole history once the ring wrapped
    o_all, _ = attend(q[0], full_k[:, 0], full_v[:, 0])
    assert not np.allclose(out[0], o_all, atol=1e-6)


def test_ring_slot_table_contiguous_history_matches_closed_form():
    w = _tiny("f32")
    for step in (0, 5, 29):
        t = int(w.decode_positions(step)[0])
        assert list(ring_slot_table(w, 0, step)) == slot_contents(t, w.sinks, w.window)


def test_stored_keys_are_rounded_rotations():
    w = _tiny("bf16")
    k, _ = ring_rows(w, 0, [0, 5, 17])
    bits = np.asarray(k, np.float32).view(np.uint32) & 0xFFFF
    assert np.all(bits == 0)        # every stored value is a bf16 value
    k0, _ = ring_rows(w, 0, [0])
    from oracle.rounding import round_bf16
    from synth import TENSOR_K
    assert np.array_equal(k0[0], round_bf16(w.rows(TENSOR_K, 0, [0])[0]))  # pos 0: no rotation


def test_pins_catch_planted_mistakes():
    rng = np.random.default_rng(6)
    q, K, V = rng.standard_normal(16), rng.standard_normal((9, 16)), rng.standard_normal((9, 16))
    want = _sdpa(q, K, V)

    def no_scale(q, K, V):
        s = K @ q
        e = np.exp(s - s.max())
        return e / e.sum() @ V

    def misindexed_values(q, K, V):
        s = K @ q / 4.0
        e = np.exp(s - s.max())
        return (e / e.sum()) @ V[::-1]

    def unnormalised(q, K, V):
        s = K @ q / 4.0
        return np.exp(s - s.max()) @ V

    for bad in (no_scale, misindexed_values, unnormalised):
        assert not np.allclose(bad(q, K, V), want, atol=1e-6), bad.__name__


@pytest.mark.parametrize("sinks,window,first", [(4, 16, 30), (0, 8, 5), (2, 64, 1), (3, 5, 0)])
def test_prefill_rows_are_windowed_causal_attention(sinks, window, first):
    """A prefill chunk's expected rows (decode steps of the workload) equal one
    masked scaled_dot_product_attention over the whole history: query j at
    t = first + j keeps the positions p <= t with p < S or p > t - W."""
    from oracle.decode import ring_prefill_expected
    T = 12
    w = RingWorkload(name="p", seed=7, batch=1, num_q_heads=4, num_kv_heads=2, head_dim=16,
                     dtype="f32", window=window, sinks=sinks, rope_base=10000.0, scale=1.0,
                     decode_steps=T, history=f"prefill:{first}")
    n = first + T
    K, V = ring_rows(w, 0, range(n))                       # [n, Hkv, d]
    Q = np.stack([ring_query(w, 0, first + j) for j in range(T)])  # [T, Hq, d]
    t = first + np.arange(T)[:, None]
    p = np.arange(n)[None, :]
    keep = (p <= t) & ((p < sinks) | (p > t - window))
    qt = torch.from_numpy(Q).permute(1, 0, 2)[None]        # [1, Hq, T, d]
    kt = torch.from_numpy(np.ascontiguousarray(K)).permute(1, 0, 2)[None].contiguous()
    vt = torch.from_numpy(np.ascontiguousarray(V)).permute(1, 0, 2)[None].contiguous()
    want = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(keep),
                                          enable_gqa=True)[0].permute(1, 0, 2).numpy()
    got, _ = ring_prefill_expected(w, 0, 0, T)
    assert np.abs(got - want).max() < 1e-12

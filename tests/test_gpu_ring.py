"""GPU parity of the ring-cache path (append + decode) against the oracle.

Bars: slot_pos bit-exact after every append; stored K rows equal the oracle's
rounded rotation (a float64 rotation computed by two libm's may land on the
other side of a rounding boundary: at most 1 ulp, in a vanishing fraction of
elements); V rows bit-exact; outputs within 1e-5 (float32 cache) or 2e-3
(bf16 cache, fp32 accumulation) max-abs of the float64 oracle.
"""

import numpy as np
import pytest
import torch

from oracle.attention import attend_heads
from oracle.decode import (ring_expected, ring_query, ring_rows, ring_slot_table)
from synth import WORKLOADS, RingWorkload

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-3}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _W(**kw):
    base = dict(name="t", seed=21, batch=2, num_q_heads=4, num_kv_heads=4, head_dim=128,
                dtype="bf16", window=300, sinks=4, rope_base=10000.0, scale=0.5,
                decode_steps=8, history="chunks:100:7")
    base.update(kw)
    return RingWorkload(**base)


def _ulps(got: np.ndarray, want: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        g = (np.asarray(got, np.float32).view(np.int32) >> 16).astype(np.int64)
        w = (np.asarray(want, np.float32).view(np.int32) >> 16).astype(np.int64)
    else:
        g = np.asarray(got, np.float32).view(np.int32).astype(np.int64)
        w = np.asarray(want, np.float32).view(np.int32).astype(np.int64)
    return np.abs(g - w)


def check_cache_rows(state, b: int, table: np.ndarray, style: str = "interleaved"):
    """Every filled slot holds the rounded rotation (K) / the raw row (V) of its position."""
    w = state.w
    filled = np.nonzero(table >= 0)[0]
    k_want, v_want = ring_rows(w, b, table[filled], style)
    k_got = state.cache.k[b][:, filled].float().cpu().numpy().transpose(1, 0, 2)
    v_got = state.cache.v[b][:, filled].float().cpu().numpy().transpose(1, 0, 2)
    assert np.array_equal(v_got, v_want.astype(np.float32))
    u = _ulps(k_got, k_want, w.dtype)
    assert u.max() <= 1, u.max()
    assert (u > 0).mean() < 1e-4


def run_and_check(w: RingWorkload, steps, style="interleaved", check_every_append=False):
    from tests.device_data import RingState
    st = RingState(w, rope_style=style)
    try:
        def after(first, n):
            if check_every_append:
                torch.cuda.synchronize()
                sp = st.cache.slot_pos.cpu().numpy()
                for b in range(w.batch):
                    last = int(first[b]) + n - 1
                    table = ring_slot_table_upto(w, b, last)
                    assert np.array_equal(sp[b], table)
        st.prefill(after)
        torch.cuda.synchronize()
        sp = st.cache.slot_pos.cpu().numpy()
        for b in range(w.batch):
            assert np.array_equal(sp[b], ring_slot_table(w, b)), b
            check_cache_rows(st, b, sp[b], style)
        for step in range(max(steps) + 1):
            inp = st.step_inputs(step)
            st.step(inp)
            if step not in steps:
                continue
            torch.cuda.synchronize()
            out = st.out.float().cpu().numpy()
            lse = st.lse.cpu().numpy()
            q_got = inp["q"][:, 0].float().cpu().numpy()
            sp = st.cache.slot_pos.cpu().numpy()
            for b in range(w.batch):
                assert np.array_equal(sp[b], ring_slot_table(w, b, step)), (b, step)
                t = int(w.decode_positions(step)[b])
                u = _ulps(q_got[b], ring_query(w, b, t, style), w.dtype)
                assert u.max() <= 1
                want, want_lse = ring_expected(w, b, step, style=style)
                err = np.abs(out[b] - want).max()
                assert err <= TOL[w.dtype], (b, step, err)
                assert np.abs(lse[b] - want_lse).max() <= 10 * TOL[w.dtype], (b, step)
        return st
    finally:
        st.close()


def ring_slot_table_upto(w, b, last):
    from oracle.ring import simulate_appends
    pos = []
    for first, n in w.history_calls():
        for p in range(int(first[b]), int(first[b]) + n):
            if p <= last:
                pos.append(p)
    return np.asarray(simulate_appends(pos, w.sinks, w.window), dtype=np.int32)


def test_tiny_ring_every_step():
    """The float32 tiny ring workload: prefill 20 tokens in one call, then 64
    decode steps, every step checked (slot_pos, rotated query, out, lse)."""
    w = WORKLOADS["tiny-ring"]
    run_and_check(w, steps=set(range(w.decode_steps)), check_every_append=True)


@pytest.mark.parametrize("kw", [
    dict(),                                                            # MHA d=128, wraps twice
    dict(num_q_heads=8, num_kv_heads=2, window=257, history="prefill:600", batch=3),  # g=4
    dict(num_q_heads=12, num_kv_heads=2, window=1000, sinks=0, history="chunks:333:4"),  # g=6
    dict(num_q_heads=6, num_kv_heads=2, head_dim=64, window=100, history="chunks:70:5"),  # g=3
    dict(num_q_heads=16, num_kv_heads=2, head_dim=64, window=64, sinks=1,
         history="chunks:50:3"),                                       # g=8, d=64
    dict(num_q_heads=4, num_kv_heads=2, head_dim=64, window=33, history="prefill:10"),  # below capacity
    dict(dtype="f32", num_q_heads=4, num_kv_heads=4, window=129, history="chunks:64:5"),
    dict(dtype="f32", num_q_heads=8, num_kv_heads=4, head_dim=64, window=50, sinks=2,
         history="chunks:40:3"),
    dict(history="sinks+window", pos0_range=(5000, 70000), window=512, batch=3),
    # positions near 2^31: the f64 angle and its reduction modulo 2 pi
    dict(history="sinks+window", pos0_range=(2_147_000_000, 2_147_480_000), window=300, batch=2,
         num_q_heads=8, num_kv_heads=2),
    dict(window=1, sinks=4, history="chunks:10:2", num_q_heads=8, num_kv_heads=2),  # W = 1
    dict(window=2, sinks=8, history="prefill:20", num_q_heads=8, num_kv_heads=2),   # S > W
])
def test_ring_variants(kw):
    w = _W(**kw)
    run_and_check(w, steps={0, 1, 5, 7}, check_every_append=True)


def test_half_rope_style():
    w = _W(num_q_heads=8, num_kv_heads=2, window=100, history="chunks:64:3")
    run_and_check(w, steps={0, 3}, style="half")


def _fresh(w):
    from tests.device_data import RingState
    return RingState(w)


def test_multi_token_call_equals_single_appends():
    """One T-token call (T > W: several tokens share a ring slot, and the call
    straddles the sink slots) leaves the same cache as T single appends."""
    w = _W(head_dim=64, window=16, sinks=4, batch=2, num_q_heads=4, num_kv_heads=2)
    a, b_ = _fresh(w), _fresh(w)
    try:
        first = np.array([2, 9], dtype=np.int64)
        T = 45
        a.append(first, T)
        for j in range(T):
            b_.append(first + j, 1)
        torch.cuda.synchronize()
        assert torch.equal(a.cache.slot_pos, b_.cache.slot_pos)
        sp = a.cache.slot_pos.cpu().numpy()
        for b in range(w.batch):
            want = ring_slot_table_upto_positions(range(int(first[b]), int(first[b]) + T), w)
            assert np.array_equal(sp[b], want)
            filled = np.nonzero(sp[b] >= 0)[0]
            assert torch.equal(a.cache.k[b][:, filled], b_.cache.k[b][:, filled])
            assert torch.equal(a.cache.v[b][:, filled], b_.cache.v[b][:, filled])
            check_cache_rows(a, b, sp[b])
    finally:
        a.close()
        b_.close()


def ring_slot_table_upto_positions(positions, w):
    from oracle.ring import simulate_appends
    return np.asarray(simulate_appends(list(positions), w.sinks, w.window), dtype=np.int32)


def test_negative_positions_are_ignored():
    """Tokens with a negative position write nothing and leave their query as is."""
    from decode_attention_fixed_amd import binding as B
    from oracle.rope import rope
    from oracle.rounding import round_bf16
    w = _W(head_dim=64, window=16, sinks=4, batch=1, num_q_heads=2, num_kv_heads=2)
    st = _fresh(w)
    try:
        g = torch.Generator().manual_seed(5)
        k, v, q = [(torch.randn(1, 8, 2, 64, generator=g) * 0.5).to(torch.bfloat16)
                   for _ in range(3)]
        qd = q.cuda()
        B.kv_append_rope(st.cache.handle, k.cuda(), v.cuda(),
                         torch.tensor([-5], dtype=torch.int32, device="cuda"), qd)
        torch.cuda.synchronize()
        want = ring_slot_table_upto_positions(range(0, 3), w)
        assert np.array_equal(st.cache.slot_pos[0].cpu().numpy(), want)
        qg = qd.float().cpu().numpy()
        for j in range(8):
            p = j - 5
            if p < 0:
                assert np.array_equal(qg[0, j], q[0, j].float().numpy())
                continue
            kr = round_bf16(rope(k[0, j].double().numpy(), p, w.rope_base))
            assert _ulps(st.cache.k[0, :, p].float().cpu().numpy(), kr, "bf16").max() <= 1
            assert torch.equal(st.cache.v[0, :, p].cpu(), v[0, j])
            qr = round_bf16(rope(q[0, j].double().numpy(), p, w.rope_base))
            assert _ulps(qg[0, j], qr, "bf16").max() <= 1
    finally:
        st.close()


def test_empty_cache_and_nan_poisoned_slots():
    """No resident row: out = 0 and lse = -inf.  Empty slots full of NaN never
    leak into the result."""
    from decode_attention_fixed_amd import binding as B
    w = _W(head_dim=128, window=200, sinks=4, batch=2, num_q_heads=8, num_kv_heads=2)
    st = _fresh(w)
    try:
        st.cache.k.fill_(float("nan"))
        st.cache.v.fill_(float("nan"))
        q = torch.randn(w.batch, w.num_q_heads, w.head_dim, device="cuda").to(torch.bfloat16)
        B.decode_attn_ring(st.cache.handle, q, st.out, st.workspace, st.lse)
        torch.cuda.synchronize()
        assert torch.all(st.out == 0)
        assert torch.all(torch.isneginf(st.lse))
        qr = st.append(np.array([0, 7]), 3, with_q=True)
        B.decode_attn_ring(st.cache.handle, qr[:, 2].contiguous(), st.out, st.workspace, st.lse)
        torch.cuda.synchronize()
        out = st.out.cpu().numpy()
        assert np.isfinite(out).all()
        for b, first in enumerate((0, 7)):
            pos = list(range(first, first + 3))
            k, v = ring_rows(w, b, pos)
            want, _ = attend_heads(ring_query(w, b, first + 2), k, v)
            assert np.abs(out[b] - want).max() <= TOL["bf16"]
    finally:
        st.close()


def test_bf16_output_and_determinism():
    from decode_attention_fixed_amd import binding as B
    w = _W(num_q_heads=8, num_kv_heads=2, window=400, history="chunks:128:4")
    st = _fresh(w)
    try:
        st.prefill()
        inp = st.step_inputs(0)
        st.step(inp)
        torch.cuda.synchronize()
        ref = st.out.clone()
        q = inp["q"][:, 0]
        for _ in range(3):
            B.decode_attn_ring(st.cache.handle, q, st.out, st.workspace, st.lse)
            torch.cuda.synchronize()
            assert torch.equal(st.out, ref)      # run-to-run bitwise identical
        o16 = torch.empty_like(st.out, dtype=torch.bfloat16)
        B.decode_attn_ring(st.cache.handle, q, o16, st.workspace, None)
        torch.cuda.synchronize()
        assert torch.equal(o16, ref.to(torch.bfloat16))   # same numbers, rounded once
    finally:
        st.close()

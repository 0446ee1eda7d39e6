"""GPU tests of the fused decode step (decode_step_ring): one call appends the
new token of every sequence and attends with its query.

Against the two-call path on an identical cache (kv_append_rope rotating a
copy of the query, then decode_attn_ring): K, V and slot_pos bit-identical
after every step, the query left unchanged, out / lse within 1e-5 (the new
token's score is summed in another order; both accumulate in float32).
Against the float64 oracle: the usual bars (slot tables exact, outputs within
2e-3 for bf16 caches, 1e-5 for float32 ones).
"""

import numpy as np
import pytest
import torch

from oracle.decode import ring_expected, ring_slot_table
from synth import RingWorkload

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-3}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _W(**kw):
    base = dict(name="s", seed=41, batch=2, num_q_heads=4, num_kv_heads=4, head_dim=128,
                dtype="bf16", window=300, sinks=4, rope_base=10000.0, scale=0.5,
                decode_steps=12, history="chunks:100:7")
    base.update(kw)
    return RingWorkload(**base)


def _log(msg):
    print(msg, flush=True)


def _two_call_step(st, inp):
    """kv_append_rope (rotating a copy of q) then decode_attn_ring."""
    from decode_attention_fixed_amd import binding as B
    q = inp["q"].clone()
    B.kv_append_rope(st.cache.handle, inp["k"], inp["v"], inp["pos"], q)
    B.decode_attn_ring(st.cache.handle, q[:, 0], st.out, st.workspace, st.lse)


def _fused_step(st, inp):
    from decode_attention_fixed_amd import binding as B
    B.decode_step_ring(st.cache.handle, inp["k"][:, 0], inp["v"][:, 0], inp["pos"],
                       inp["q"][:, 0], st.out, st.workspace, st.lse)


def _pair(w):
    """Two caches with the same history; rows never written hold the same
    (zero) bytes in both, so whole caches can be compared."""
    from tests.device_data import RingState
    a, b = RingState(w), RingState(w)
    for st in (a, b):
        st.cache.k.zero_()
        st.cache.v.zero_()
        st.prefill()
    torch.cuda.synchronize()
    return a, b


def _compare(a, b, step):
    assert torch.equal(a.cache.slot_pos, b.cache.slot_pos), step
    assert torch.equal(a.cache.k, b.cache.k), step
    assert torch.equal(a.cache.v, b.cache.v), step
    assert (a.out - b.out).abs().max().item() <= 1e-5, step
    la, lb = a.lse, b.lse
    fin = torch.isfinite(la)
    assert torch.equal(fin, torch.isfinite(lb)), step
    if fin.any():
        assert (la[fin] - lb[fin]).abs().max().item() <= 1e-5, step


@pytest.mark.parametrize("kw", [
    dict(),                                                                  # g=1, wraps
    dict(num_q_heads=16, num_kv_heads=4, window=257, history="prefill:600", batch=3),  # g=4
    dict(num_q_heads=12, num_kv_heads=2, window=1000, sinks=0, history="chunks:333:4"),  # g=6
    dict(num_q_heads=16, num_kv_heads=2, window=64, sinks=1, history="chunks:50:3"),    # g=8
    dict(num_q_heads=8, num_kv_heads=2, window=64, sinks=4, history="prefill:1"),  # into sinks
    dict(batch=1, num_q_heads=8, num_kv_heads=2, window=20000, sinks=4,
         history="prefill:25000", decode_steps=4),                          # many splits + merge
    dict(dtype="f32", head_dim=64, num_q_heads=8, num_kv_heads=4, window=50, sinks=2,
         history="chunks:40:3"),                                            # two-launch path
    dict(window=1, sinks=4, history="chunks:10:2", num_q_heads=8, num_kv_heads=2),  # W = 1
    dict(window=2, sinks=8, history="prefill:3", num_q_heads=8, num_kv_heads=2),    # S > W
])
def test_fused_step_equals_two_calls(kw):
    w = _W(**kw)
    a, b = _pair(w)
    try:
        for step in range(w.decode_steps):
            inp = a.step_inputs(step)
            q_before = inp["q"].clone()
            _two_call_step(a, inp)
            _fused_step(b, inp)
            torch.cuda.synchronize()
            assert torch.equal(inp["q"], q_before)   # the fused step leaves q as given
            _compare(a, b, step)
        _log(f"{kw}: {w.decode_steps} steps, cache bit-identical")
    finally:
        a.close()
        b.close()


@pytest.mark.parametrize("kw", [
    dict(),                                                                  # g=1, wraps
    dict(num_q_heads=16, num_kv_heads=4, window=257, history="prefill:600", batch=3),  # g=4
    dict(batch=1, num_q_heads=8, num_kv_heads=2, window=20000, sinks=4,
         history="prefill:25000", decode_steps=4),                          # many splits + merge
    dict(window=2, sinks=8, history="prefill:3", num_q_heads=8, num_kv_heads=2),    # S > W
])
def test_fused_step_equals_two_calls_i8(kw):
    """int8 caches: the fused step quantises the new rows exactly as the int8
    append does (codes and scales bit-identical).  Outputs: with g <= 2 both
    paths weigh rows in float32 (1e-5 as above); with g >= 3 P*V runs on the
    matrix core with fp16 weights (11 significant bits) while the fused step
    adds the new token in float32 at the merge, so the two differ by up to
    2^-11 of the new token's share of the output: 1e-3."""
    w = _W(cache="i8", **kw)
    tol = 1e-5 if w.num_q_heads // w.num_kv_heads <= 2 else 1e-3
    a, b = _pair(w)
    try:
        for step in range(w.decode_steps):
            inp = a.step_inputs(step)
            q_before = inp["q"].clone()
            _two_call_step(a, inp)
            _fused_step(b, inp)
            torch.cuda.synchronize()
            assert torch.equal(inp["q"], q_before)
            assert torch.equal(a.cache.slot_pos, b.cache.slot_pos), step
            assert torch.equal(a.cache.k, b.cache.k), step
            assert torch.equal(a.cache.v, b.cache.v), step
            assert (a.out - b.out).abs().max().item() <= tol, step
            fin = torch.isfinite(a.lse)
            assert torch.equal(fin, torch.isfinite(b.lse)), step
            if fin.any():
                assert (a.lse[fin] - b.lse[fin]).abs().max().item() <= 1e-5, step
        _log(f"i8 {kw}: {w.decode_steps} steps, cache bit-identical")
    finally:
        a.close()
        b.close()


def test_fused_step_negative_position():
    """A sequence whose position is negative appends nothing and attends with
    its query as given, in both paths."""
    w = _W(num_q_heads=8, num_kv_heads=2, window=64, history="chunks:40:2", batch=3)
    a, b = _pair(w)
    try:
        for step in range(3):
            inp = a.step_inputs(step)
            inp["pos"][1] = -7
            _two_call_step(a, inp)
            _fused_step(b, inp)
            torch.cuda.synchronize()
            _compare(a, b, step)
    finally:
        a.close()
        b.close()


@pytest.mark.parametrize("kw", [
    dict(num_q_heads=16, num_kv_heads=4, window=512, history="sinks+window",
         pos0_range=(3000, 50000), batch=4),
    dict(num_q_heads=12, num_kv_heads=2, window=700, history="chunks:256:4"),
    dict(num_q_heads=8, num_kv_heads=2, window=300, history="sinks+window",
         pos0_range=(2_147_000_000, 2_147_480_000)),                        # positions near 2^31
])
def test_fused_step_oracle(kw):
    """Decode steps run through decode_step_ring only, against the oracle."""
    from tests.device_data import RingState
    w = _W(**kw)
    st = RingState(w)
    try:
        st.prefill()
        for step in range(w.decode_steps):
            _fused_step(st, st.step_inputs(step))
            if step not in (0, 1, w.decode_steps - 1):
                continue
            torch.cuda.synchronize()
            sp = st.cache.slot_pos.cpu().numpy()
            out = st.out.float().cpu().numpy()
            lse = st.lse.cpu().numpy()
            for bb in range(w.batch):
                assert np.array_equal(sp[bb], ring_slot_table(w, bb, step)), (bb, step)
                want, want_lse = ring_expected(w, bb, step)
                assert np.abs(out[bb] - want).max() <= TOL[w.dtype], (bb, step)
                assert np.abs(lse[bb] - want_lse).max() <= 10 * TOL[w.dtype], (bb, step)
    finally:
        st.close()

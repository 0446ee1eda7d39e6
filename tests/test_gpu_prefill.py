"""GPU tests of the chunked prefill (prefill_attn_ring).

Bars: every query row of the chunk within 2e-3 max-abs of the float64 oracle
(row j of a chunk = decode step j of the workload, bf16 cache, fp32
accumulation, P * V in fp16), lse within 2e-2; after the call the cache (K,
V, slot_pos) bit-identical to kv_append_rope of the same chunk; the query
left unchanged.
"""

import numpy as np
import pytest
import torch

from oracle.attention import attend_heads
from oracle.decode import ring_prefill_expected
from synth import RingWorkload

pytestmark = pytest.mark.gpu

TOL = 2e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _W(**kw):
    base = dict(name="pf", seed=51, batch=2, num_q_heads=4, num_kv_heads=4, head_dim=128,
                dtype="bf16", window=300, sinks=4, rope_base=10000.0, scale=0.5,
                decode_steps=64, history="chunks:100:7")
    base.update(kw)
    return RingWorkload(**base)


def _log(msg):
    print(msg, flush=True)


def _pair(w):
    from tests.device_data import RingState
    a, b = RingState(w), RingState(w)
    for st in (a, b):
        st.cache.k.zero_()
        st.cache.v.zero_()
        st.prefill()
    torch.cuda.synchronize()
    return a, b


@pytest.mark.parametrize("kw", [
    dict(),                                                                    # g=1, T=64
    dict(num_q_heads=16, num_kv_heads=4, window=257, history="prefill:600", batch=3,
         decode_steps=100),                                                    # g=4
    dict(num_q_heads=12, num_kv_heads=2, window=1000, sinks=0, history="chunks:333:4",
         decode_steps=37),                                                     # g=6, ragged block
    dict(num_q_heads=16, num_kv_heads=2, window=64, sinks=1, history="chunks:50:3",
         decode_steps=200),                                                    # g=8, T > W
    dict(num_q_heads=8, num_kv_heads=2, window=64, sinks=4, history="prefill:1",
         decode_steps=20),                                                     # into the sinks
    dict(num_q_heads=4, num_kv_heads=2, decode_steps=1),                       # g=2, T=1
    dict(num_q_heads=6, num_kv_heads=2, window=128, history="sinks+window",
         pos0_range=(3000, 9000), decode_steps=45),                            # g=3
])
def test_prefill_matches_oracle_and_append(kw):
    from decode_attention_fixed_amd import binding as B
    w = _W(**kw)
    T = w.decode_steps
    a, b = _pair(w)
    try:
        inp = a.chunk_inputs(0, T)
        q_before = inp["q"].clone()
        out = torch.empty(w.batch, T, w.num_q_heads, w.head_dim, device="cuda")
        lse = torch.empty(w.batch, T, w.num_q_heads, device="cuda")
        a.prefill_chunk(inp, out, lse)
        B.kv_append_rope(b.cache.handle, inp["k"], inp["v"], inp["pos"])
        torch.cuda.synchronize()
        assert torch.equal(inp["q"], q_before)
        assert torch.equal(a.cache.slot_pos, b.cache.slot_pos)
        assert torch.equal(a.cache.k, b.cache.k)
        assert torch.equal(a.cache.v, b.cache.v)
        o = out.cpu().numpy()
        l = lse.cpu().numpy()
        worst = 0.0
        for bb in range(w.batch):
            want, want_lse = ring_prefill_expected(w, bb, 0, T)
            err = float(np.abs(o[bb] - want).max())
            worst = max(worst, err)
            assert err <= TOL, (bb, err)
            assert np.abs(l[bb] - want_lse).max() <= 2e-2, bb
        _log(f"{kw}: T={T} max-abs error {worst:.2e}")
    finally:
        a.close()
        b.close()


def test_prefill_negative_positions_and_empty_cache():
    """A chunk starting at position -3 on an empty cache: rows at negative
    positions give out = 0, lse = -inf; the others attend the chunk's tokens
    from position 0 up to their own (and nothing else)."""
    from tests.device_data import RingState
    w = _W(num_q_heads=8, num_kv_heads=2, window=16, sinks=2, batch=1, history="prefill:0")
    st = RingState(w)
    try:
        T = 24
        g = torch.Generator().manual_seed(9)
        k, v, q = [(torch.randn(1, T, h, 128, generator=g) * 0.5).to(torch.bfloat16).cuda()
                   for h in (2, 2, 8)]
        pos = torch.tensor([-3], dtype=torch.int32, device="cuda")
        out = torch.empty(1, T, 8, 128, device="cuda")
        lse = torch.empty(1, T, 8, device="cuda")
        st.prefill_chunk(dict(k=k, v=v, q=q, pos=pos), out, lse)
        torch.cuda.synchronize()
        from oracle.rope import rope
        from oracle.rounding import round_bf16
        kr = [round_bf16(rope(k[0, j].double().cpu().numpy(), j - 3, w.rope_base))
              for j in range(T)]
        for j in range(T):
            t = j - 3
            if t < 0:
                assert torch.all(out[0, j] == 0) and torch.all(torch.isneginf(lse[0, j]))
                continue
            keep = [i for i in range(3, j + 1) if (i - 3) < w.sinks or (i - 3) > t - w.window]
            K = np.stack([kr[i] for i in keep])
            V = np.stack([v[0, i].double().cpu().numpy() for i in keep])
            qr = round_bf16(rope(q[0, j].double().cpu().numpy(), t, w.rope_base))
            want, want_lse = attend_heads(qr, K, V)
            assert np.abs(out[0, j].cpu().numpy() - want).max() <= TOL, j
            assert np.abs(lse[0, j].cpu().numpy() - want_lse).max() <= 2e-2, j
    finally:
        st.close()


def test_prefill_chunks_continue_the_ring():
    """Two chunks in a row (the second attends the first through the ring),
    sampled rows against the oracle."""
    from tests.device_data import RingState
    w = _W(num_q_heads=16, num_kv_heads=4, window=200, history="chunks:64:2", decode_steps=160)
    st = RingState(w)
    try:
        st.prefill()
        for first, n in ((0, 90), (90, 70)):
            inp = st.chunk_inputs(first, n)
            out = torch.empty(w.batch, n, w.num_q_heads, w.head_dim, device="cuda")
            st.prefill_chunk(inp, out)
            torch.cuda.synchronize()
            o = out.cpu().numpy()
            rows = [0, 1, n // 2, n - 1]
            for bb in range(w.batch):
                want, _ = ring_prefill_expected(w, bb, first, n, rows=rows)
                assert np.abs(o[bb][rows] - want).max() <= TOL, (first, bb)
    finally:
        st.close()

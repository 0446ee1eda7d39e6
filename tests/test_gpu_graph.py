"""HIP-graph capture of the library's calls (torch.cuda.CUDAGraph over the
launches on the current stream).

Every entry point of a decode step only launches kernels on its stream, so a
step can be captured once and replayed; positions live in device memory and
swa_pos_advance moves them on inside the graph.  Each replay is compared bit
for bit with the same calls issued eagerly on a twin cache (the same kernels
on the same bytes), with eager work and synchronisations between the replays,
so a node that only worked on its first replay would show.
"""

import pytest
import torch

from synth import TENSOR_K, TENSOR_Q, TENSOR_V, PoolWorkload, RingWorkload

pytestmark = pytest.mark.gpu

REPLAYS = 5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _ring(**kw):
    base = dict(name="g", seed=61, batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128,
                dtype="bf16", window=300, sinks=4, rope_base=10000.0, scale=0.5,
                decode_steps=REPLAYS, history="chunks:100:5")
    base.update(kw)
    return RingWorkload(**base)


def _twins(w):
    from tests.device_data import RingState
    a, b = RingState(w), RingState(w)
    for st in (a, b):
        st.cache.k.zero_()   # slots never written hold the same bytes in both
        st.cache.v.zero_()
        st.prefill()
    torch.cuda.synchronize()
    return a, b


def _same_ring(a, b, s):
    assert torch.equal(a.out, b.out), s
    assert torch.equal(a.lse, b.lse), s
    assert torch.equal(a.cache.slot_pos, b.cache.slot_pos), s
    assert torch.equal(a.cache.k, b.cache.k), s
    assert torch.equal(a.cache.v, b.cache.v), s


@pytest.mark.parametrize("kw,fused", [
    (dict(), True),                                   # one fused launch per step
    (dict(), False),                                  # append, then decode
    (dict(cache="i8"), False),                        # int8 rows
    (dict(cache="i8"), True),                         # int8 rows, fused step
    (dict(positions="cache"), True),                  # cache position shifting
    (dict(dtype="f32", head_dim=64, num_q_heads=4, num_kv_heads=4, window=40), True),
])
def test_ring_step_replays(kw, fused):
    from decode_attention_fixed_amd import binding as B
    w = _ring(**kw)
    eager, graphed = _twins(w)
    try:
        inputs = [eager.step_inputs(s) for s in range(REPLAYS)]
        # step 0 eagerly on the eager twin first: every kernel is loaded
        eager.step({**inputs[0], "q": inputs[0]["q"].clone()}, fused=fused)
        gk = inputs[0]["k"].clone()
        gv = inputs[0]["v"].clone()
        gq = inputs[0]["q"].clone()
        gpos = inputs[0]["pos"].clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            graphed.step(dict(k=gk, v=gv, q=gq, pos=gpos), fused=fused)
            B.pos_advance(gpos, 1)
        for s in range(REPLAYS):
            if s > 0:
                eager.step({**inputs[s], "q": inputs[s]["q"].clone()}, fused=fused)
            # eager work between replays: this step's rows into the graph's inputs
            gk.copy_(inputs[s]["k"])
            gv.copy_(inputs[s]["v"])
            gq.copy_(inputs[s]["q"])
            assert torch.equal(gpos, inputs[s]["pos"]), s
            g.replay()
            torch.cuda.synchronize()
            _same_ring(eager, graphed, s)
        assert torch.equal(gpos, inputs[-1]["pos"] + 1)
    finally:
        eager.close()
        graphed.close()


@pytest.mark.parametrize("cache", ["", "i8"])
def test_pool_decode_replays(cache):
    from decode_attention_fixed_amd import binding as B
    from tests.device_data import PagedState
    w = PoolWorkload(name="gp", seed=62, batch=2, num_q_heads=6, num_kv_heads=1, head_dim=128,
                     dtype="bf16", block_size=64, logical_blocks=64, pool_slots=20,
                     rope_base=10000.0, scale=0.5, decode_steps=REPLAYS, cache=cache)
    st = PagedState(w)
    st.k_pool.fill_(255 if cache else float("nan"))  # rows nobody writes: never read
    st.v_pool.fill_(255 if cache else float("nan"))
    st.fill()
    qs = [st.step_query(s) for s in range(REPLAYS)]
    gq = qs[0].clone()
    out = torch.empty_like(st.out)
    lse = torch.empty_like(st.lse)
    ws = torch.empty_like(st.workspace)
    st.step(qs[0])  # loads every kernel
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.decode_attn_paged(st.desc, gq, st.k_pool, st.v_pool, st.block_table, st.seq_lens,
                            st.block_valid, out, ws, lse)
    for s in range(REPLAYS):
        st.step(qs[s])
        gq.copy_(qs[s])
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, st.out), s
        assert torch.equal(lse, st.lse), s


def test_prefill_replays():
    """prefill_attn_ring (rotation, attention, append: three launches) captured
    once and replayed on successive chunks, positions moved on by the chunk
    length inside the graph."""
    from decode_attention_fixed_amd import binding as B
    from tests.device_data import to_device
    T = 32
    w = _ring(history="chunks:64:4", window=160)
    eager, graphed = _twins(w)
    try:
        hq, hkv, d = w.num_q_heads, w.num_kv_heads, w.head_dim
        pos0 = w.decode_start.astype("int32")

        def chunk(c):
            first = pos0 + c * T
            k = eager._rows(TENSOR_K, first, T)
            v = eager._rows(TENSOR_V, first, T)
            q = eager._rows(TENSOR_Q, first, T)
            return (to_device(k, w.dtype), to_device(v, w.dtype), to_device(q, w.dtype),
                    torch.from_numpy(first.astype("int32")).cuda())

        chunks = [chunk(c) for c in range(REPLAYS)]
        n = B.prefill_attn_workspace_bytes(w.batch, hq, hkv, d, T)
        ws_e = torch.empty(n, dtype=torch.uint8, device="cuda")
        ws_g = torch.empty(n, dtype=torch.uint8, device="cuda")
        out_e = torch.empty((w.batch, T, hq, d), dtype=torch.float32, device="cuda")
        out_g = torch.empty_like(out_e)
        lse_e = torch.empty((w.batch, T, hq), dtype=torch.float32, device="cuda")
        lse_g = torch.empty_like(lse_e)
        k0, v0, q0, p0 = chunks[0]
        B.prefill_attn_ring(eager.cache.handle, k0, v0, p0, q0, out_e, ws_e, lse_e)
        gk, gv, gq, gpos = k0.clone(), v0.clone(), q0.clone(), p0.clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            B.prefill_attn_ring(graphed.cache.handle, gk, gv, gpos, gq, out_g, ws_g, lse_g)
            B.pos_advance(gpos, T)
        for c in range(REPLAYS):
            k, v, q, p = chunks[c]
            if c > 0:
                B.prefill_attn_ring(eager.cache.handle, k, v, p, q, out_e, ws_e, lse_e)
            gk.copy_(k)
            gv.copy_(v)
            gq.copy_(q)
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out_g, out_e), c
            assert torch.equal(lse_g, lse_e), c
            assert torch.equal(graphed.cache.slot_pos, eager.cache.slot_pos), c
            assert torch.equal(graphed.cache.k, eager.cache.k), c
            assert torch.equal(graphed.cache.v, eager.cache.v), c
    finally:
        eager.close()
        graphed.close()


def test_pos_advance_values():
    """pos += delta on the device, clamped to the int32 range."""
    from decode_attention_fixed_amd import binding as B
    big = 2**31 - 1
    vals = [0, -5, 7, big - 1, big, -(2**31), -(2**31) + 2]
    pos = torch.tensor(vals, dtype=torch.int32, device="cuda")
    B.pos_advance(pos, 3)
    torch.cuda.synchronize()
    want = [min(max(v + 3, -(2**31)), big) for v in vals]
    assert pos.cpu().tolist() == want
    B.pos_advance(pos, -10)
    torch.cuda.synchronize()
    assert pos.cpu().tolist() == [min(max(v - 10, -(2**31)), big) for v in want]
    empty = torch.empty(0, dtype=torch.int32, device="cuda")
    B.pos_advance(empty, 1)  # nothing to do

"""GPU parity of the host-pool pager ([pool] "paging", LRU residency) against
the oracle.

For every decode step: the logical block in each slot (host state) equals the
oracle's LRU simulation bit for bit; the device validity bytes equal the
oracle's visible set; the attention output over the pool equals attention
over exactly the visible blocks, within the bf16 bar.  At the end every
filled slot's pool block holds the host store's bytes of its logical block,
bit for bit (paging moves bytes and changes none).

Pool rows that the pager has not written hold NaN, so a slot read before its
copy lands, or after its eviction, would show.
"""

import numpy as np
import pytest
import torch

from oracle.decode import pager_expected, pager_schedule
from oracle.paging import LruPool
from synth import PagerWorkload, workload

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-3
TOL_F32 = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _pager(**kw):
    base = dict(name="pg", seed=61, batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128,
                dtype="bf16", block_size=64, logical_blocks=48, pool_slots=12, rope_base=10000.0,
                scale=0.5, decode_steps=10, prefill_blocks=4, window_blocks=2, focus_blocks=3,
                focus_drift=2, revisits=2)
    base.update(kw)
    return PagerWorkload(**base)


def _state(w):
    from tests.device_data import PagerState
    st = PagerState(w)
    st.k_pool.fill_(float("nan"))
    st.v_pool.fill_(float("nan"))
    st.fill_host()
    st.reset()
    return st


def _check_pool_bytes(st, w, slots_by_seq):
    """Every filled slot's pool block equals the host store's block."""
    kp = st.k_pool.cpu()
    vp = st.v_pool.cpu()
    for b in range(w.batch):
        for j, blk in enumerate(slots_by_seq[b]):
            if blk < 0:
                continue
            ph = int(w.slot_phys[b, j])
            assert torch.equal(kp[ph].view(torch.int16), st.host_k[b, blk].view(torch.int16)) \
                if kp.dtype == torch.bfloat16 else torch.equal(kp[ph], st.host_k[b, blk])
            assert torch.equal(vp[ph].view(torch.int16), st.host_v[b, blk].view(torch.int16)) \
                if vp.dtype == torch.bfloat16 else torch.equal(vp[ph], st.host_v[b, blk])


def _run(w, st, steps_to_check, copy_stream=None, tol=TOL_BF16):
    """copy_stream: a stream for every copy, None (the attention stream), or
    a list of those used in turn."""
    sched = [pager_schedule(w, b) for b in range(w.batch)]
    cycle = copy_stream if isinstance(copy_stream, list) else [copy_stream]
    st.warm(cycle[0])
    for step in range(w.decode_steps):
        if step + 1 < w.decode_steps:
            st.advance(st.step_requests(step + 1), cycle[step % len(cycle)])
        st.decode(st.step_query(step))
        torch.cuda.synchronize()
        valid = st.block_valid.cpu().numpy()
        for b in range(w.batch):
            visible, slots = sched[b][0][step], sched[b][1][step]
            got_slots = st.slot_blocks(b)
            assert got_slots == slots, (step, b)
            vis = set(visible)
            want_valid = np.array([1 if (s >= 0 and s in vis) else 0 for s in slots],
                                  dtype=np.uint8)
            assert np.array_equal(valid[b], want_valid), (step, b)
        if step in steps_to_check:
            out = st.out.cpu().numpy()
            lse = st.lse.cpu().numpy()
            for b in range(w.batch):
                want, want_lse = pager_expected(w, b, step, sched[b][0][step])
                err = float(np.abs(out[b] - want).max())
                assert err <= tol, (step, b, err)
                assert float(np.abs(lse[b] - want_lse).max()) <= 1e-4
    st.commit()
    torch.cuda.synchronize()
    _check_pool_bytes(st, w, [st.slot_blocks(b) for b in range(w.batch)])


@pytest.mark.parametrize("copies", ["attention-stream", "side-stream", "alternating"])
def test_pager_small(copies):
    w = _pager()
    st = _state(w)
    try:
        side = torch.cuda.Stream()
        cs = {"attention-stream": None, "side-stream": side, "alternating": [None, side]}[copies]
        _run(w, st, set(range(w.decode_steps)), cs)
    finally:
        st.close()


@pytest.mark.parametrize("kw,tol", [
    (dict(dtype="f32", head_dim=64, num_q_heads=4, num_kv_heads=4, block_size=16), TOL_F32),
    (dict(num_q_heads=24, num_kv_heads=4, pool_slots=15, prefill_blocks=5, seed=62,
          logical_blocks=80, decode_steps=12), TOL_BF16),
])
def test_pager_shapes(kw, tol):
    w = _pager(**kw)
    st = _state(w)
    try:
        _run(w, st, {0, w.decode_steps // 2, w.decode_steps - 1}, torch.cuda.Stream(), tol)
    finally:
        st.close()


def test_pager_refusal_changes_nothing():
    """A request that needs more than the empty plus evictable slots is
    refused on the host, launches nothing and leaves the state as it was."""
    from decode_attention_fixed_amd.binding import SWA_ERR_INVALID_ARG, SwaError
    w = _pager(batch=1, pool_slots=6, logical_blocks=16)
    st = _state(w)
    try:
        pool = LruPool(w.pool_slots)
        for req in ([0, 1, 2], [0, 1, 2, 3, 4, 5]):
            st.advance([req])
            pool.advance(req)
        before = st.slot_blocks(0)
        with pytest.raises(SwaError) as e:
            st.advance([[6]])  # all six resident blocks were named by the previous request
        assert e.value.code == SWA_ERR_INVALID_ARG
        assert st.slot_blocks(0) == before
        for req in ([3], [3, 6, 6, 7]):  # then 0, 1, 2, 4, 5 are evictable; repeats count once
            st.advance([req])
            pool.advance(req)
        st.commit()
        pool.commit()
        torch.cuda.synchronize()
        assert st.slot_blocks(0) == pool.slot_block
        valid = st.block_valid.cpu().numpy()[0]
        assert valid.tolist() == [1 if b >= 0 else 0 for b in pool.slot_block]
        _check_pool_bytes(st, w, [pool.slot_block])
    finally:
        st.close()


def test_pager_full_size():
    """The long-pool-swap workload at full size: 256K-token context in host
    memory, 1152 device slots, LRU paging; sampled steps against the oracle,
    every step's slot map and validity bytes exact."""
    w = workload("long-pool-swap")
    st = _state(w)
    try:
        n = w.decode_steps
        _run(w, st, {0, 1, n // 2, n - 1}, torch.cuda.Stream())
    finally:
        st.close()

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

The paging step folded into the decode (swa_pager_stage, then
swa_pager_decode copying the staged blocks in its merge launch) is checked
the same way against the oracle's fused schedule: a step attends the blocks
resident when it starts, and after it every resident block is valid.
"""

import numpy as np
import pytest
import torch

from oracle.decode import pager_expected, pager_schedule, pager_schedule_fused
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


def _run_fused(w, st, steps_to_check, tol=TOL_BF16, seqs=None):
    """stage(N_{t+1}); decode(t) for every step; outputs checked on the
    sequences `seqs` (all: None)."""
    sched = [pager_schedule_fused(w, b) for b in range(w.batch)]
    st.warm(None)
    for step in range(w.decode_steps):
        if step + 1 < w.decode_steps:
            st.stage(st.step_requests(step + 1))
        st.fused_decode(st.step_query(step))
        torch.cuda.synchronize()
        valid = st.block_valid.cpu().numpy()
        for b in range(w.batch):
            visible, slots = sched[b][0][step], sched[b][1][step]
            assert st.slot_blocks(b) == slots, (step, b)
            want_valid = np.array([1 if s >= 0 else 0 for s in slots], dtype=np.uint8)
            assert np.array_equal(valid[b], want_valid), (step, b)
        if step in steps_to_check:
            out = st.out.cpu().numpy()
            lse = st.lse.cpu().numpy()
            for b in (range(w.batch) if seqs is None else seqs):
                want, want_lse = pager_expected(w, b, step, sched[b][0][step])
                err = float(np.abs(out[b] - want).max())
                assert err <= tol, (step, b, err)
                assert float(np.abs(lse[b] - want_lse).max()) <= 1e-4
    torch.cuda.synchronize()
    _check_pool_bytes(st, w, [st.slot_blocks(b) for b in range(w.batch)])


@pytest.mark.parametrize("kw,tol", [
    (dict(), TOL_BF16),                                              # bf16, g = 4
    (dict(num_q_heads=24, num_kv_heads=4, pool_slots=15, prefill_blocks=5, seed=62,
          logical_blocks=80, decode_steps=12), TOL_BF16),            # g = 6
    (dict(dtype="f32", head_dim=64, num_q_heads=4, num_kv_heads=4, block_size=16),
     TOL_F32),                                                       # copies after the decode
])
def test_pager_fused_step(kw, tol):
    w = _pager(**kw)
    st = _state(w)
    try:
        _run_fused(w, st, set(range(w.decode_steps)), tol)
    finally:
        st.close()


def test_pager_fused_step_wide_grid():
    """A pool of 1M rows of capacity takes the 512 x 4-wave grid; a fused step
    gives the workgroups of 8 CUs to the fetch, so the attention runs on 496
    workgroups (shares by division, not by shift) and the merge finds the
    owners of 496 shares."""
    w = _pager(batch=8, num_q_heads=4, num_kv_heads=1, pool_slots=2048, logical_blocks=3000,
               prefill_blocks=128, window_blocks=16, focus_blocks=16, focus_drift=8, revisits=16,
               decode_steps=3, seed=66)
    assert w.batch * w.num_kv_heads * w.pool_slots * w.block_size >= 512 * 2048
    st = _state(w)
    try:
        # step 0 stages 53 blocks (folded), step 1 stages 75 (more than a
        # folded step takes: launches of their own after the decode)
        _run_fused(w, st, {0, 1}, seqs=[0, 5])
    finally:
        st.close()


def test_pager_fused_step_many_blocks():
    """More staged blocks than one merge launch takes (64): they are copied
    by launches after the decode, with the same result."""
    w = _pager(batch=8, pool_slots=80, logical_blocks=120, focus_blocks=30, focus_drift=30,
               revisits=4, decode_steps=6, seed=64)
    st = _state(w)
    try:
        st.warm(None)
        n = st.stage(st.step_requests(1))
        assert n > 64, n
        st.fused_decode(st.step_query(0))
        torch.cuda.synchronize()
        sched = [pager_schedule_fused(w, b) for b in range(w.batch)]
        valid = st.block_valid.cpu().numpy()
        out = st.out.cpu().numpy()
        for b in range(w.batch):
            assert st.slot_blocks(b) == sched[b][1][0]
            assert np.array_equal(valid[b], np.array([1 if s >= 0 else 0 for s in sched[b][1][0]],
                                                     dtype=np.uint8))
            want, _ = pager_expected(w, b, 0, sched[b][0][0])
            assert float(np.abs(out[b] - want).max()) <= TOL_BF16
        _check_pool_bytes(st, w, [st.slot_blocks(b) for b in range(w.batch)])
    finally:
        st.close()


def test_pager_stage_order_rules():
    """A second stage before the decode, an advance while a stage is pending,
    and a stage while an advance's copies are pending are refused, launching
    nothing; commit runs a pending stage's copies without an attention."""
    from decode_attention_fixed_amd.binding import SWA_ERR_INVALID_ARG, SwaError
    w = _pager(batch=1, decode_steps=4)
    st = _state(w)
    try:
        st.warm(None)
        assert st.stage(st.step_requests(1)) >= 0
        with pytest.raises(SwaError) as e:
            st.stage(st.step_requests(2))
        assert e.value.code == SWA_ERR_INVALID_ARG
        with pytest.raises(SwaError) as e:
            st.advance(st.step_requests(2))
        assert e.value.code == SWA_ERR_INVALID_ARG
        st.commit()
        torch.cuda.synchronize()
        slots = st.slot_blocks(0)
        valid = st.block_valid.cpu().numpy()[0]
        assert list(valid) == [1 if s >= 0 else 0 for s in slots]
        _check_pool_bytes(st, w, [slots])
        st.advance(st.step_requests(2))
        with pytest.raises(SwaError) as e:
            st.stage(st.step_requests(3))
        assert e.value.code == SWA_ERR_INVALID_ARG
        with pytest.raises(SwaError) as e:
            st.fused_decode(st.step_query(1))
        assert e.value.code == SWA_ERR_INVALID_ARG
    finally:
        st.close()



def test_pager_decode_workspace_too_small():
    """swa_pager_decode refuses a workspace below swa_pager_workspace_bytes
    (the decode's own size is not enough: the staging area follows it),
    launching nothing and leaving the stage pending."""
    from decode_attention_fixed_amd import binding as B
    from decode_attention_fixed_amd.binding import SWA_ERR_WORKSPACE, SwaError
    w = _pager(batch=2, decode_steps=4)
    st = _state(w)
    try:
        st.warm(None)
        need = B.swa_pager_workspace_bytes(st.handle, w.num_q_heads)
        dec = B.decode_attn_workspace_bytes(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                            w.pool_slots * w.block_size)
        assert need > dec
        n = st.stage(st.step_requests(1))
        assert n > 0
        small = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
        pool_k = st.k_pool.clone()
        valid = st.block_valid.clone()
        with pytest.raises(SwaError) as e:
            B.swa_pager_decode(st.handle, st.desc, st.step_query(0), st.k_pool, st.v_pool,
                               st.block_table, st.seq_lens, st.block_valid, st.out, small,
                               st.lse)
        assert e.value.code == SWA_ERR_WORKSPACE
        torch.cuda.synchronize()
        assert torch.equal(pool_k, st.k_pool) and torch.equal(valid, st.block_valid)
        # the stage still stands: the decode with the right workspace copies it
        st.fused_decode(st.step_query(0))
        torch.cuda.synchronize()
        sched = [pager_schedule_fused(w, b) for b in range(w.batch)]
        for b in range(w.batch):
            assert st.slot_blocks(b) == sched[b][1][0]
        _check_pool_bytes(st, w, [st.slot_blocks(b) for b in range(w.batch)])
    finally:
        st.close()

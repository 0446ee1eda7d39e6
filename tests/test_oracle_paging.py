"""Pins for oracle/paging.py (LRU residency of a fixed block pool, [pool]
"residency policy")."""

import random

import pytest

from oracle.paging import LruPool, PoolRefused


def lru_most_recent(requests, capacity):
    """The defining property of LRU, computed straight from the request
    string: the `capacity` most recently used distinct blocks."""
    seen = []
    for b in reversed(list(requests)):
        if b not in seen:
            seen.append(b)
        if len(seen) == capacity:
            break
    return set(seen)


@pytest.mark.parametrize("capacity", [2, 3, 5, 8])
@pytest.mark.parametrize("universe", [4, 10, 40])
def test_single_block_requests_hold_most_recent(capacity, universe):
    rng = random.Random(capacity * 100 + universe)
    pool = LruPool(capacity)
    trace = []
    for _ in range(300):
        b = rng.randrange(universe)
        trace.append(b)
        pool.request([b])
        assert pool.resident() == lru_most_recent(trace, capacity)
        assert pool.visible() == pool.resident()


def test_inclusion_property():
    """A pool of C slots holds a subset of what a pool of C + 1 slots holds."""
    rng = random.Random(7)
    pools = [LruPool(c) for c in range(2, 9)]
    for _ in range(400):
        b = rng.randrange(20)
        for p in pools:
            p.request([b])
        for small, big in zip(pools, pools[1:]):
            assert small.resident() <= big.resident()


@pytest.mark.parametrize("k,chunks_held", [(4, 3), (64, 18)])
def test_chunked_streaming(k, chunks_held):
    """Streaming a history in consecutive chunks of k blocks through C = m*k
    slots leaves the last m chunks, block j in slot j mod C (free slots fill
    in order; afterwards the oldest chunk's slots are reused in slot order)."""
    cap = k * chunks_held
    pool = LruPool(cap)
    n_chunks = 3 * chunks_held + 1
    for c in range(n_chunks):
        pool.advance(range(c * k, (c + 1) * k))
        held = set(range(max(0, (c + 1 - chunks_held) * k), (c + 1) * k))
        pool.commit()
        assert pool.resident() == held
        for j in held:
            assert pool.slot_block[j % cap] == j


def test_in_flight_visibility():
    """Between advance and commit the copies are invisible and their slots'
    previous blocks are gone."""
    pool = LruPool(4)
    pool.request([0, 1])
    pool.request([2, 3])
    loads = pool.advance([4, 5])
    assert [b for _, b in loads] == [4, 5]
    # victims: blocks 0 and 1 (oldest, unprotected), slots 0 and 1
    assert sorted(pool.evicting) == [(0, 0), (1, 1)]
    assert pool.visible() == {2, 3}
    pool.commit()
    assert pool.visible() == {2, 3, 4, 5}


def test_previous_request_protected():
    """With two slots and alternating requests the previous block survives."""
    pool = LruPool(2)
    pool.request([0])
    pool.request([1])
    pool.advance([2])      # evicts 0 (1 was the previous request)
    assert pool.resident() == {1, 2}
    one = LruPool(1)
    one.request([0])
    with pytest.raises(PoolRefused):
        one.request([1])   # 0 is protected as the previous request: refused


def test_refusal_leaves_state():
    pool = LruPool(3)
    pool.request([0, 1, 2])
    before = (list(pool.slot_block), dict(pool.last_use), pool.clock, set(pool.prev))
    with pytest.raises(PoolRefused):
        pool.advance([3])  # all three resident blocks were named by the previous request
    assert (list(pool.slot_block), dict(pool.last_use), pool.clock, set(pool.prev)) == before
    pool.advance([0])      # a request within the resident set is fine
    pool.advance([3])      # now 1 and 2 are evictable: 1 is at the lower slot
    assert pool.resident() == {0, 2, 3}


def test_random_trace_invariants():
    """Brute-force checks over random multi-block traces: every requested
    block is resident afterwards, no block of the previous or current request
    is evicted, the victim is always a least recently used evictable block,
    and refusals happen exactly when misses exceed free + evictable slots."""
    rng = random.Random(11)
    for trial in range(30):
        cap = rng.randrange(3, 12)
        pool = LruPool(cap)
        prev = set()
        for _ in range(60):
            req = [rng.randrange(3 * cap) for _ in range(rng.randrange(0, cap))]
            reqset = set(req)
            resident = pool.resident()
            missing = reqset - resident
            free = pool.slot_block.count(-1)
            evictable = [b for b in resident if b not in reqset | prev]
            last_use = dict(pool.last_use)
            before = list(pool.slot_block)
            if len(missing) > free + len(evictable):
                with pytest.raises(PoolRefused):
                    pool.advance(req)
                assert pool.slot_block == before
                continue
            pool.advance(req)
            assert reqset <= pool.resident()
            evicted = resident - pool.resident()
            assert not (evicted & (reqset | prev))
            assert len(evicted) == max(0, len(missing) - free)
            if evicted:
                kept = [b for b in evictable if b not in evicted]
                assert max(last_use[b] for b in evicted) <= min(
                    (last_use[b] for b in kept), default=1 << 30)
            assert pool.visible() == (pool.resident() - missing)
            prev = reqset


@pytest.mark.parametrize("seed,slots", [(61, 12), (62, 15), (63, 10)])
def test_fused_schedule_against_the_advance_schedule(seed, slots):
    """oracle/decode.py's two pager schedules, pinned against each other and
    the LRU pool: with the paging step folded into the decode, step t sees
    every block its request names, exactly what the advance-then-decode
    order shows it plus the blocks that step t + 1's request evicts, and the
    pool after serving step t + 1's request is the same in both orders."""
    from oracle.decode import pager_schedule, pager_schedule_fused
    from synth import PagerWorkload
    w = PagerWorkload(name="pg", seed=seed, batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128,
                      dtype="bf16", block_size=64, logical_blocks=48, pool_slots=slots,
                      rope_base=10000.0, scale=0.5, decode_steps=12, prefill_blocks=4,
                      window_blocks=2, focus_blocks=3, focus_drift=2, revisits=2)
    for b in range(w.batch):
        vis_a, slots_a = pager_schedule(w, b)
        vis_f, slots_f = pager_schedule_fused(w, b)
        assert slots_a == slots_f
        evicted_total = 0
        for t in range(w.decode_steps):
            named = set(int(x) for x in w.step_request(b, t))
            assert named <= set(vis_f[t]), (b, t)
            assert set(vis_a[t]) <= set(vis_f[t]), (b, t)
            before = set(slots_f[t - 1]) - {-1} if t > 0 else set(vis_f[0])
            assert set(vis_f[t]) == before, (b, t)  # everything resident at its start
            if t + 1 < w.decode_steps:  # (the last step serves no next request)
                evicted = before - (set(slots_f[t]) - {-1})
                assert set(vis_f[t]) - set(vis_a[t]) == evicted, (b, t)
                evicted_total += len(evicted)
        assert evicted_total > 0  # the case evicts blocks

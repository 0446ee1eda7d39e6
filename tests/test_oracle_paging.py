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

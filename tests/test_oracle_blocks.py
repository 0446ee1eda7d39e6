"""Pins for oracle/blocks.py (refcounted blocks, prefix sharing, copy-on-write;
[share] §3.2, §5.1, §6.1)."""

import random

import pytest

from oracle.blocks import BlockManager, BlocksExhausted


def _check_invariants(m: BlockManager):
    count = [0] * m.num_blocks
    for table in m.tables.values():
        for b in table:
            count[b] += 1
    assert count == m.ref                               # refcount = table entries naming it
    for seq, table in m.tables.items():
        assert len(table) == -(-m.lens[seq] // m.block_size)   # ceil(len / bs) blocks
    assert m.free_count() == sum(1 for c in count if c == 0)


def test_page_prefix_example():
    """[share] §3.2: a 2000-token system prompt and 100 concurrent requests:
    without sharing the prompt's KV is stored 100 times, with sharing once.
    With 16-token blocks (§5.2) that is 125 blocks instead of 12,500."""
    bs, n = 16, 100
    shared = BlockManager(20000, bs)
    shared.allocate("prompt", 2000)
    for i in range(n):
        shared.share_prefix("prompt", i, 2000)
    assert shared.num_blocks - shared.free_count() == 125
    private = BlockManager(20000, bs)
    for i in range(n):
        private.allocate(i, 2000)
    assert private.num_blocks - private.free_count() == 12500
    _check_invariants(shared)
    # each request continues on its own: the first append at 2000 = 125 * 16
    # takes a fresh block (no copy needed, the shared blocks are full)
    for i in range(n):
        _, copied = shared.append_token(i)
        assert copied is None
    assert shared.num_blocks - shared.free_count() == 125 + n
    _check_invariants(shared)


def test_copy_on_write_partial_block():
    """A shared, partly filled last block is copied before either sharer
    writes into it; the other sequence keeps seeing its own rows."""
    m = BlockManager(16, 4)
    m.allocate("a", 6)                 # blocks 0, 1 (block 1 half full)
    m.share_prefix("a", "b", 6)
    assert m.ref[:2] == [2, 2]
    row, copied = m.append_token("b")  # b writes row 2 of block 1: copy first
    assert copied == (1, 2, 2) and row == (2, 2)
    assert m.ref[:3] == [2, 1, 1]
    row, copied = m.append_token("a")  # a's block 1 is private again: no copy
    assert copied is None and row == (1, 2)
    assert m.read("a") == [("a", i) for i in range(7)]
    assert m.read("b") == [("a", i) for i in range(6)] + [("b", 6)]
    _check_invariants(m)


def test_free_keeps_shared_blocks():
    """[share] §6.1: ending a sequence whose blocks are still shared only
    drops its references; the other sequence's prefix survives."""
    m = BlockManager(8, 4)
    m.allocate("a", 8)
    m.share_prefix("a", "b", 8)
    m.free("a")
    assert m.free_count() == 6
    assert m.read("b") == [("a", i) for i in range(8)]
    m.allocate("c", 16)                # takes the 4 blocks nobody holds
    assert m.read("b") == [("a", i) for i in range(8)]
    with pytest.raises(BlocksExhausted):
        m.allocate("d", 12)
    _check_invariants(m)


def test_lowest_free_block_first():
    m = BlockManager(6, 4)
    m.allocate("a", 4)
    m.allocate("b", 8)
    assert m.tables == {"a": [0], "b": [1, 2]}
    m.free("a")
    m.allocate("c", 12)
    assert m.tables["c"] == [0, 3, 4]


def _random_run(m, rng, steps=400, seqs=8):
    """Random interleaving of the four operations; returns each live
    sequence's expected history (tags in order)."""
    hist = {}
    for _ in range(steps):
        op = rng.random()
        live = list(hist)
        try:
            if op < 0.15 or not live:
                s = max(hist, default=-1) + 1
                n = rng.randrange(0, 3 * m.block_size)
                m.allocate(s, n)
                hist[s] = [(s, i) for i in range(n)]
            elif op < 0.3 and len(live) < seqs:
                src = rng.choice(live)
                n = rng.randrange(0, m.lens[src] + 1)
                s = max(hist) + 1
                m.share_prefix(src, s, n)
                hist[s] = hist[src][:n]
            elif op < 0.4:
                s = rng.choice(live)
                m.free(s)
                del hist[s]
            else:
                s = rng.choice(live)
                m.append_token(s)
                hist[s].append((s, m.lens[s] - 1))
        except BlocksExhausted:
            pass
        _check_invariants(m)
    return hist


@pytest.mark.parametrize("seed", range(6))
def test_isolation_random(seed):
    rng = random.Random(seed)
    m = BlockManager(40, rng.choice([2, 4, 16]))
    hist = _random_run(m, rng)
    for s, h in hist.items():
        assert m.read(s) == h


class _NoCopyOnWrite(BlockManager):
    """Planted mistake: writes into shared blocks in place."""

    def append_token(self, seq, tag=None):
        table = self.tables.setdefault(seq, [])
        n = self.lens.get(seq, 0)
        if n % self.block_size == 0:
            table.append(self._take())
        row = (table[-1], n % self.block_size)
        self.rows[row] = tag if tag is not None else (seq, n)
        self.lens[seq] = n + 1
        return row, None


class _FreeIgnoresRefs(BlockManager):
    """Planted mistake: the §6.1 bug, freeing without looking at references."""

    def free(self, seq):
        for b in self.tables.pop(seq, []):
            self.ref[b] = 0
            for i in range(self.block_size):
                self.rows.pop((b, i), None)
        self.lens.pop(seq, None)


@pytest.mark.parametrize("cls", [_NoCopyOnWrite, _FreeIgnoresRefs])
def test_planted_mistakes_break_isolation(cls):
    broken = 0
    for seed in range(6):
        rng = random.Random(seed)
        m = cls(40, 4)
        hist = {}
        try:
            hist = _random_run(m, rng)
            broken += any(m.read(s) != h for s, h in hist.items())
        except AssertionError:
            broken += 1
    assert broken > 0

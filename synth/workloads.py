"""The decode workloads as seeded, synthetic input recipes.

Three kinds of workload:

* RingWorkload   - a sink + sliding-window ring cache that is filled by a list
  of append calls and then decoded one token per step (each step appends the
  new token and attends).
* PagedWorkload  - a block-table KV pool (16-token blocks) with ragged lengths
  and a common prompt prefix shared through identical block ids; read-only
  decode steps with a fresh query per step.  PagedAppendWorkload: the same
  contents grown through a block manager, one new token per sequence and step.
* PoolWorkload   - one long logical context split in 64-token blocks, of which
  only a fixed-size pool of slots is resident; a per-slot validity mask marks
  the filled slots; read-only decode steps.
* PagerWorkload  - the same long context held whole in host memory, with a
  device pool of slots filled on demand: a string of block requests (a
  chunked prefill streaming the history, then one request per decode step:
  the window's blocks, a drifting focus region and a few random revisits).

Everything here is an input: shapes, draws, lengths, start positions, which
logical block sits in which pool slot, and the physical block ids.  How a
position maps to a cache slot or a pool row is the method's business and is
not computed here.
"""

from __future__ import annotations

import dataclasses
import functools

import numpy as np

from .draws import (CHUNK, SHARED_SEQUENCE, TENSOR_K, TENSOR_Q, TENSOR_V, draw_rows,
                    draw_rows_parallel)

# Sub-stream ids for the structural draws (kept apart from the row tensors).
_S_POS0 = 100
_S_LENGTHS = 101
_S_PERM = 102
_S_RESIDENT = 103
_S_SUBSET = 104
_S_PLACE = 105
_S_FOCUS = 106
_S_REVISIT = 107


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(stream)])


@dataclasses.dataclass(frozen=True)
class RingWorkload:
    name: str
    seed: int
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str              # "f32" or "bf16": cache, new-token and query dtype
    window: int             # W
    sinks: int              # S
    rope_base: float
    scale: float            # raw rows are N(0,1) * scale
    decode_steps: int
    history: str            # "prefill:<T>" | "chunks:<T>:<N>" | "sinks+window"
    pos0_range: tuple = (0, 0)   # used by "sinks+window": decode start ~ U[lo, hi)
    chunk: int = 0          # prefill workloads: decode steps taken `chunk` tokens per call
    cache: str = ""         # "i8": int8 cache rows (inputs stay `dtype`); "": same as dtype
    positions: str = ""     # "cache": positions inside the attention are cache indices

    kind = "ring"

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def slots(self) -> int:
        return self.sinks + self.window

    @functools.cached_property
    def decode_start(self) -> np.ndarray:
        """Absolute position of the first decode token, per sequence (int64 [B])."""
        kind, *args = self.history.split(":")
        if kind == "prefill":
            return np.full(self.batch, int(args[0]), dtype=np.int64)
        if kind == "chunks":
            return np.full(self.batch, int(args[0]) * int(args[1]), dtype=np.int64)
        if kind == "sinks+window":
            lo, hi = self.pos0_range
            return _rng(self.seed, _S_POS0).integers(lo, hi, size=self.batch).astype(np.int64)
        raise ValueError(self.history)

    def history_calls(self) -> list:
        """Append calls that build the cache before decoding.

        Each call is (first_position int64 [B], n_tokens): sequence b appends
        positions first_position[b] .. first_position[b] + n_tokens - 1."""
        kind, *args = self.history.split(":")
        if kind == "prefill":
            return [(np.zeros(self.batch, dtype=np.int64), int(args[0]))]
        if kind == "chunks":
            t, n = int(args[0]), int(args[1])
            return [(np.full(self.batch, c * t, dtype=np.int64), t) for c in range(n)]
        if kind == "sinks+window":
            start = self.decode_start
            return [(np.zeros(self.batch, dtype=np.int64), self.sinks),
                    (start - self.window, self.window)]
        raise ValueError(self.history)

    def decode_positions(self, step: int) -> np.ndarray:
        return self.decode_start + int(step)

    # -- rows -----------------------------------------------------------------
    def rows(self, tensor: int, b: int, positions) -> np.ndarray:
        heads = self.num_q_heads if tensor == TENSOR_Q else self.num_kv_heads
        return draw_rows(self.seed, tensor, b, positions, heads, self.head_dim, self.scale,
                         self.dtype)

    def rows_range(self, tensor: int, b: int, start: int, count: int, out=None) -> np.ndarray:
        heads = self.num_q_heads if tensor == TENSOR_Q else self.num_kv_heads
        return draw_rows_parallel(self.seed, tensor, b, start, count, heads, self.head_dim,
                                  self.scale, self.dtype, out=out)

    def kv_bytes_per_token(self) -> int:
        if self.cache == "i8":  # codes plus one float32 scale per row
            return 2 * self.num_kv_heads * (self.head_dim + 4)
        e = 4 if self.dtype == "f32" else 2
        return 2 * self.num_kv_heads * self.head_dim * e


@dataclasses.dataclass(frozen=True)
class PagedWorkload:
    name: str
    seed: int
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str
    block_size: int
    len_range: tuple        # inclusive [lo, hi]
    shared_prefix: int      # tokens shared by every sequence (multiple of block_size)
    scale: float
    decode_steps: int
    cache: str = ""         # "i8": int8 pool rows (inputs stay `dtype`)

    kind = "paged"

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def max_blocks(self) -> int:
        return -(-self.len_range[1] // self.block_size)

    @functools.cached_property
    def lengths(self) -> np.ndarray:
        lo, hi = self.len_range
        return _rng(self.seed, _S_LENGTHS).integers(lo, hi, size=self.batch,
                                                    endpoint=True).astype(np.int64)

    @functools.cached_property
    def shared_blocks(self) -> int:
        assert self.shared_prefix % self.block_size == 0
        return self.shared_prefix // self.block_size

    @functools.cached_property
    def logical_blocks(self) -> list:
        """Per sequence: list of unique-block ids for its logical blocks.

        Unique ids 0 .. shared_blocks-1 are the shared prefix blocks; private
        blocks follow, sequence by sequence."""
        nxt = self.shared_blocks
        out = []
        for b in range(self.batch):
            nb = -(-int(self.lengths[b]) // self.block_size)
            ids = list(range(min(nb, self.shared_blocks)))
            n_priv = max(0, nb - self.shared_blocks)
            ids += list(range(nxt, nxt + n_priv))
            nxt += n_priv
            out.append(np.asarray(ids, dtype=np.int64))
        return out

    @functools.cached_property
    def num_unique_blocks(self) -> int:
        return self.shared_blocks + sum(max(0, len(x) - self.shared_blocks)
                                        for x in self.logical_blocks)

    @functools.cached_property
    def physical_of_unique(self) -> np.ndarray:
        """Seeded permutation: unique block id -> physical block id."""
        return _rng(self.seed, _S_PERM).permutation(self.num_unique_blocks).astype(np.int64)

    @functools.cached_property
    def block_table(self) -> np.ndarray:
        """int32 [B, max_blocks]; entries past a sequence's last block are -1."""
        bt = np.full((self.batch, self.max_blocks), -1, dtype=np.int32)
        for b, ids in enumerate(self.logical_blocks):
            bt[b, :len(ids)] = self.physical_of_unique[ids]
        return bt

    def row_source(self, b: int, positions) -> tuple:
        """(sequence stream, position) pairs that hold the raw rows of sequence b."""
        pos = np.asarray(positions, dtype=np.int64)
        seq = np.where(pos < self.shared_prefix, SHARED_SEQUENCE, b)
        return seq, pos

    def rows(self, tensor: int, b: int, positions) -> np.ndarray:
        """Raw K/V rows of sequence b at logical positions (shared prefix aware)."""
        seq, pos = self.row_source(b, positions)
        out = np.empty((pos.size, self.num_kv_heads, self.head_dim), dtype=np.float32)
        for s in np.unique(seq):
            sel = np.nonzero(seq == s)[0]
            out[sel] = draw_rows(self.seed, tensor, int(s), pos[sel], self.num_kv_heads,
                                 self.head_dim, self.scale, self.dtype)
        return out

    def query(self, b: int, step: int) -> np.ndarray:
        return draw_rows(self.seed, TENSOR_Q, b, [step], self.num_q_heads, self.head_dim,
                         self.scale, self.dtype)[0]

    def kv_bytes_per_token(self) -> int:
        if getattr(self, "cache", "") == "i8":  # codes plus one float32 scale per row
            return 2 * self.num_kv_heads * (self.head_dim + 4)
        return 2 * self.num_kv_heads * self.head_dim * 2


@dataclasses.dataclass(frozen=True)
class PagedAppendWorkload(PagedWorkload):
    """The paged workload built and grown through a block manager: the shared
    prefix is written once and shared by reference, every sequence's own
    tokens are appended, and each decode step first appends one new token per
    sequence (at position lengths[b] + step, drawn from the sequence's own
    stream) and then attends over all of them."""

    kind = "paged-append"

    def row_source(self, b: int, positions) -> tuple:
        """Rows of sequence b: the shared stream for the part of the prefix it
        shares when built (its first min(lengths[b], shared_prefix) tokens),
        its own stream for everything after, appended tokens included."""
        pos = np.asarray(positions, dtype=np.int64)
        shared = min(int(self.lengths[b]), self.shared_prefix)
        return np.where(pos < shared, SHARED_SEQUENCE, b), pos


@dataclasses.dataclass(frozen=True)
class PoolWorkload:
    name: str
    seed: int
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str
    block_size: int         # tokens per block (and per pool slot)
    logical_blocks: int     # context length / block_size
    pool_slots: int         # resident slots per sequence
    rope_base: float
    scale: float
    decode_steps: int
    cache: str = ""         # "i8": int8 pool rows (inputs stay `dtype`)

    kind = "pool"

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def context(self) -> int:
        return self.logical_blocks * self.block_size

    @functools.cached_property
    def slot_blocks(self) -> np.ndarray:
        """int64 [B, pool_slots]: logical block held by each slot, -1 if empty.

        Each logical block is resident with probability pool_slots /
        logical_blocks; when more are drawn than there are slots, a seeded
        subset of pool_slots blocks is kept; the resident blocks are placed in
        seeded slots."""
        p = self.pool_slots / self.logical_blocks
        res = _rng(self.seed, _S_RESIDENT).random((self.batch, self.logical_blocks)) < p
        sub = _rng(self.seed, _S_SUBSET)
        place = _rng(self.seed, _S_PLACE)
        out = np.full((self.batch, self.pool_slots), -1, dtype=np.int64)
        for b in range(self.batch):
            blocks = np.nonzero(res[b])[0]
            if blocks.size > self.pool_slots:
                blocks = np.sort(sub.choice(blocks, self.pool_slots, replace=False))
            slots = place.permutation(self.pool_slots)[:blocks.size]
            out[b, slots] = blocks
        return out

    @functools.cached_property
    def block_valid(self) -> np.ndarray:
        return (self.slot_blocks >= 0).astype(np.uint8)

    @functools.cached_property
    def block_table(self) -> np.ndarray:
        """int32 [B, pool_slots]: slot -> physical block in a pool of B*pool_slots."""
        perm = _rng(self.seed, _S_PERM).permutation(self.batch * self.pool_slots)
        return perm.reshape(self.batch, self.pool_slots).astype(np.int32)

    def resident_positions(self, b: int) -> np.ndarray:
        """Logical positions held by sequence b's filled slots, in slot order."""
        blocks = self.slot_blocks[b][self.slot_blocks[b] >= 0]
        return (blocks[:, None] * self.block_size
                + np.arange(self.block_size)[None, :]).reshape(-1)

    def rows(self, tensor: int, b: int, positions) -> np.ndarray:
        return draw_rows(self.seed, tensor, b, positions, self.num_kv_heads, self.head_dim,
                         self.scale, self.dtype)

    def query(self, b: int, step: int) -> np.ndarray:
        """Query of decode step `step`; taken as already rotated at the position
        one past the context (an isotropic draw is rotation invariant)."""
        return draw_rows(self.seed, TENSOR_Q, b, [step], self.num_q_heads, self.head_dim,
                         self.scale, self.dtype)[0]

    def kv_bytes_per_token(self) -> int:
        if getattr(self, "cache", "") == "i8":  # codes plus one float32 scale per row
            return 2 * self.num_kv_heads * (self.head_dim + 4)
        return 2 * self.num_kv_heads * self.head_dim * 2


@dataclasses.dataclass(frozen=True)
class PagerWorkload:
    name: str
    seed: int
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str
    block_size: int         # tokens per block
    logical_blocks: int     # blocks of each sequence's history (all in host memory)
    pool_slots: int         # device slots per sequence
    rope_base: float
    scale: float
    decode_steps: int
    prefill_blocks: int     # blocks per request while the history streams in
    window_blocks: int      # the last blocks of the history, named by every step
    focus_blocks: int       # consecutive blocks around a focus that drifts forward
    focus_drift: int        # the focus moves U{0..focus_drift} blocks per step
    revisits: int           # uniformly drawn earlier blocks per step

    kind = "pager"

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def context(self) -> int:
        return self.logical_blocks * self.block_size

    @functools.cached_property
    def slot_phys(self) -> np.ndarray:
        """int32 [B, pool_slots]: device pool block behind each slot (a seeded
        permutation of the B * pool_slots pool blocks)."""
        perm = _rng(self.seed, _S_PERM).permutation(self.batch * self.pool_slots)
        return perm.reshape(self.batch, self.pool_slots).astype(np.int32)

    def prefill_requests(self) -> list:
        """Requests of the history streaming in: consecutive chunks of
        prefill_blocks blocks, the same for every sequence."""
        n, k = self.logical_blocks, self.prefill_blocks
        return [list(range(c, min(c + k, n))) for c in range(0, n, k)]

    @functools.cached_property
    def _focus(self) -> np.ndarray:
        """int64 [B, steps]: first block of each step's focus region."""
        g = _rng(self.seed, _S_FOCUS)
        hi = self.logical_blocks - self.window_blocks - self.focus_blocks
        start = g.integers(0, max(1, hi // 2), size=self.batch)
        drift = g.integers(0, self.focus_drift + 1, size=(self.batch, self.decode_steps))
        drift[:, 0] = 0
        return np.minimum(start[:, None] + np.cumsum(drift, axis=1), hi)

    @functools.cached_property
    def _revisits(self) -> np.ndarray:
        g = _rng(self.seed, _S_REVISIT)
        hi = self.logical_blocks - self.window_blocks
        return g.integers(0, hi, size=(self.batch, self.decode_steps, self.revisits))

    def step_request(self, b: int, step: int) -> list:
        """Blocks decode step `step` of sequence b asks for: the window's
        blocks, then the focus region, then the revisits (duplicates kept
        once, at their first place)."""
        n = self.logical_blocks
        window = range(n - self.window_blocks, n)
        f = int(self._focus[b, step])
        focus = range(f, f + self.focus_blocks)
        req = list(window) + list(focus) + [int(x) for x in self._revisits[b, step]]
        return list(dict.fromkeys(req))

    def rows(self, tensor: int, b: int, positions) -> np.ndarray:
        return draw_rows(self.seed, tensor, b, positions, self.num_kv_heads, self.head_dim,
                         self.scale, self.dtype)

    def query(self, b: int, step: int) -> np.ndarray:
        """Query of decode step `step`, taken as already rotated (an isotropic
        draw is rotation invariant)."""
        return draw_rows(self.seed, TENSOR_Q, b, [step], self.num_q_heads, self.head_dim,
                         self.scale, self.dtype)[0]

    def kv_bytes_per_token(self) -> int:
        if getattr(self, "cache", "") == "i8":  # codes plus one float32 scale per row
            return 2 * self.num_kv_heads * (self.head_dim + 4)
        return 2 * self.num_kv_heads * self.head_dim * 2


WORKLOADS = {
    "tiny-ring": RingWorkload(
        name="tiny-ring", seed=1, batch=1, num_q_heads=4, num_kv_heads=4, head_dim=64,
        dtype="f32", window=16, sinks=4, rope_base=10000.0, scale=1.0, decode_steps=64,
        history="prefill:20"),
    "mha-ring": RingWorkload(
        name="mha-ring", seed=2, batch=8, num_q_heads=32, num_kv_heads=32, head_dim=128,
        dtype="bf16", window=4096, sinks=4, rope_base=10000.0, scale=0.5, decode_steps=256,
        history="chunks:256:32"),
    "gqa-ring": RingWorkload(
        name="gqa-ring", seed=3, batch=64, num_q_heads=32, num_kv_heads=8, head_dim=128,
        dtype="bf16", window=4096, sinks=4, rope_base=10000.0, scale=0.5, decode_steps=128,
        history="sinks+window", pos0_range=(4096, 65536)),
    # Chunked prefill on the two ring caches: the tokens after the history
    # arrive 256 per sequence per call (chunks of 128-256 tokens).
    "mha-prefill": RingWorkload(
        name="mha-prefill", seed=2, batch=8, num_q_heads=32, num_kv_heads=32, head_dim=128,
        dtype="bf16", window=4096, sinks=4, rope_base=10000.0, scale=0.5, decode_steps=1024,
        history="chunks:256:32", chunk=256),
    "gqa-prefill": RingWorkload(
        name="gqa-prefill", seed=3, batch=64, num_q_heads=32, num_kv_heads=8, head_dim=128,
        dtype="bf16", window=4096, sinks=4, rope_base=10000.0, scale=0.5, decode_steps=512,
        history="sinks+window", pos0_range=(4096, 65536), chunk=256),
    "paged": PagedWorkload(
        name="paged", seed=4, batch=32, num_q_heads=32, num_kv_heads=8, head_dim=128,
        dtype="bf16", block_size=16, len_range=(1024, 32768), shared_prefix=2000, scale=0.5,
        decode_steps=128),
    # mha-ring with StreamingLLM cache position shifting ([sink]).
    "mha-ring-shift": RingWorkload(
        name="mha-ring-shift", seed=2, batch=8, num_q_heads=32, num_kv_heads=32, head_dim=128,
        dtype="bf16", window=4096, sinks=4, rope_base=10000.0, scale=0.5, decode_steps=256,
        history="chunks:256:32", positions="cache"),
    # The same workloads over int8 caches ([kvc] §5.1): codes plus one
    # float32 scale per row, quantised when written.
    "mha-ring-i8": RingWorkload(
        name="mha-ring-i8", seed=2, batch=8, num_q_heads=32, num_kv_heads=32, head_dim=128,
        dtype="bf16", window=4096, sinks=4, rope_base=10000.0, scale=0.5, decode_steps=256,
        history="chunks:256:32", cache="i8"),
    "gqa-ring-i8": RingWorkload(
        name="gqa-ring-i8", seed=3, batch=64, num_q_heads=32, num_kv_heads=8, head_dim=128,
        dtype="bf16", window=4096, sinks=4, rope_base=10000.0, scale=0.5, decode_steps=128,
        history="sinks+window", pos0_range=(4096, 65536), cache="i8"),
    "paged-i8": PagedWorkload(
        name="paged-i8", seed=4, batch=32, num_q_heads=32, num_kv_heads=8, head_dim=128,
        dtype="bf16", block_size=16, len_range=(1024, 32768), shared_prefix=2000, scale=0.5,
        decode_steps=128, cache="i8"),
    "long-pool-b16-i8": PoolWorkload(
        name="long-pool-b16-i8", seed=5, batch=16, num_q_heads=24, num_kv_heads=4, head_dim=128,
        dtype="bf16", block_size=64, logical_blocks=4096, pool_slots=1152,
        rope_base=10000.0, scale=0.5, decode_steps=128, cache="i8"),
    "paged-append": PagedAppendWorkload(
        name="paged-append", seed=4, batch=32, num_q_heads=32, num_kv_heads=8, head_dim=128,
        dtype="bf16", block_size=16, len_range=(1024, 32768), shared_prefix=2000, scale=0.5,
        decode_steps=128),
    "long-pool-b1": PoolWorkload(
        name="long-pool-b1", seed=5, batch=1, num_q_heads=24, num_kv_heads=4, head_dim=128,
        dtype="bf16", block_size=64, logical_blocks=4096, pool_slots=1152,
        rope_base=10000.0, scale=0.5, decode_steps=128),
    "long-pool-b16": PoolWorkload(
        name="long-pool-b16", seed=5, batch=16, num_q_heads=24, num_kv_heads=4, head_dim=128,
        dtype="bf16", block_size=64, logical_blocks=4096, pool_slots=1152,
        rope_base=10000.0, scale=0.5, decode_steps=128),
    # The long-pool-b1 context held whole in host memory: 1152 device slots
    # filled on demand (LRU), a 4096-token window named by every step.
    "long-pool-swap": PagerWorkload(
        name="long-pool-swap", seed=6, batch=1, num_q_heads=24, num_kv_heads=4, head_dim=128,
        dtype="bf16", block_size=64, logical_blocks=4096, pool_slots=1152,
        rope_base=10000.0, scale=0.5, decode_steps=128, prefill_blocks=64, window_blocks=64,
        focus_blocks=32, focus_drift=3, revisits=4),
}


def workload(name: str):
    return WORKLOADS[name]


__all__ = ["RingWorkload", "PagedWorkload", "PagedAppendWorkload", "PoolWorkload", "PagerWorkload",
           "WORKLOADS", "workload", "CHUNK",
           "TENSOR_K", "TENSOR_V", "TENSOR_Q"]

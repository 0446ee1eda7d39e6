"""Expected decode outputs of the synthetic workloads, from the full history.

Nothing here uses a cache slot, a ring pointer or a block table: the resident
set is written down from its definition and the rows are regenerated from
the synthetic history, so the GPU cache layout is checked, not assumed.

Ring workloads (sink + sliding window, [sink] cache formula, [ring] §2.2):
  at decode position t the query attends R(t) = sinks united with the last W
  positions, the new token included (each step appends, then attends, as the
  [ring] demo does, §4.3).  Cached K rows carry RoPE at their absolute
  position, rounded to the storage dtype ([pool] "bake RoPE into K"); V rows
  are stored as given; the query is rotated at t and stored the same way.
Cache position shifting ([sink]): the same resident set, with each key and
  the query rotated at their index in the cache instead of their position.
Chunked prefill on a ring ([pool] "paging", chunks of 128-256 tokens): a
  chunk of T new tokens at positions p0 .. p0 + T - 1; query row j is exactly
  decode step j of the same workload (position p0 + j attends R(p0 + j) after
  the tokens before it were appended), so the expected rows are the decode
  steps' outputs.
Paged workloads (block table with a shared prefix, [share] §3.1-§3.2):
  plain causal attention over all len_b tokens of sequence b; K rows are used
  as given (no RoPE on this workload).  Grown by appends ([share] §5.1), step
  s first appends the token at position len_b + s, then attends.
int8 caches ([kvc] §5.1, oracle/quant.py): every stored row is quantised
  on its own (absmax scale); attention reads code * scale.
Pool workloads (fixed pool + validity mask, [pool] "paging" and "mask"):
  attention over exactly the tokens of the resident blocks; absent blocks
  are as if they did not exist.  Resident K rows carry RoPE at their
  absolute position; the query is taken as given (already rotated).
Pager workloads ([pool] "paging", LRU residency): the blocks a decode step
  sees are those the LRU pool (oracle/paging.py) holds at that moment, with
  the copies for the next step in flight; attention over their tokens as for
  the pool workloads.
"""

from __future__ import annotations

import numpy as np

from synth import TENSOR_K, TENSOR_Q, TENSOR_V

from .attention import attend_heads
from .paging import LruPool
from .quant import quantize_dequantize
from .ring import resident_positions, simulate_appends
from .rope import rope
from .rounding import round_store


def stored_rows(w, k_rot, v):
    """What the cache holds, as float64: int8 caches hold every row quantised
    with its own scale (oracle/quant.py; K from its float64 rotation, V from
    its given values); other caches hold K rounded to the storage dtype and
    V as given."""
    if getattr(w, "cache", "") == "i8":
        return quantize_dequantize(k_rot), quantize_dequantize(np.asarray(v, dtype=np.float64))
    return round_store(k_rot, w.dtype), np.asarray(v, dtype=np.float64)


def ring_rows(w, b: int, positions, style: str = "interleaved"):
    """Cached (K, V) rows of sequence b at absolute positions: K rotated, then
    stored (rounded, or quantised for int8 caches)."""
    pos = np.asarray(positions, dtype=np.int64)
    k_raw = w.rows(TENSOR_K, b, pos)
    v = w.rows(TENSOR_V, b, pos)
    return stored_rows(w, rope(k_raw, pos[:, None], w.rope_base, style), v)


def ring_query(w, b: int, t: int, style: str = "interleaved") -> np.ndarray:
    """Query of sequence b at decode position t, rotated at t and rounded [Hq, d]."""
    q_raw = w.rows(TENSOR_Q, b, [t])[0]
    return round_store(rope(q_raw, t, w.rope_base, style), w.dtype)


def ring_expected(w, b: int, step: int, scale=None, style: str = "interleaved"):
    """(out [Hq, d], lse [Hq]) of decode step `step` for sequence b."""
    t = int(w.decode_positions(step)[b])
    pos = resident_positions(t, w.sinks, w.window)
    k, v = ring_rows(w, b, pos, style)
    return attend_heads(ring_query(w, b, t, style), k, v, scale)


def ring_cache_positions(t: int, sinks: int, window: int) -> dict:
    """Position in the cache of every position held after positions 0..t were
    appended ([sink] "cache position shifting"): the cache is the sinks
    followed by the recent window, in order, and a key's position is its
    index in that sequence; the query, the newest key, has the last index."""
    return {p: c for c, p in enumerate(resident_positions(t, sinks, window))}


def ring_shifted_expected(w, b: int, step: int, scale=None, style: str = "interleaved"):
    """(out [Hq, d], lse [Hq]) of decode step `step` with positions taken in
    the cache ([sink]: the window's positions are moved left inside the
    attention so that their distance to the sinks stays within the window):
    every key is rotated at its cache position and the query at its own, at
    read time, in float64 from the rows as given (keys are not stored
    rotated in this variant)."""
    t = int(w.decode_positions(step)[b])
    cpos = ring_cache_positions(t, w.sinks, w.window)
    pos = np.asarray(sorted(cpos), dtype=np.int64)
    c = np.asarray([cpos[p] for p in pos], dtype=np.int64)
    k = rope(w.rows(TENSOR_K, b, pos), c[:, None], w.rope_base, style)
    v = w.rows(TENSOR_V, b, pos).astype(np.float64)
    q = rope(w.rows(TENSOR_Q, b, [t])[0], cpos[t], w.rope_base, style)
    return attend_heads(q, k, v, scale)


def ring_prefill_expected(w, b: int, first_step: int, n_tokens: int, scale=None,
                          style: str = "interleaved", rows=None):
    """(out [n, Hq, d], lse [n, Hq]) of a prefill chunk made of decode steps
    first_step .. first_step + n - 1 of sequence b; `rows` restricts to a
    subset of the chunk's rows (indices into the chunk)."""
    idx = range(n_tokens) if rows is None else rows
    res = [ring_expected(w, b, first_step + j, scale, style) for j in idx]
    return np.stack([r[0] for r in res]), np.stack([r[1] for r in res])


def ring_appended_positions(w, b: int, through_step: int | None = None) -> list:
    """Every position appended to sequence b, in call order: the history calls,
    then one token per decode step up to and including `through_step`."""
    out = []
    for first, n in w.history_calls():
        out.extend(range(int(first[b]), int(first[b]) + n))
    if through_step is not None:
        start = int(w.decode_start[b])
        out.extend(range(start, start + through_step + 1))
    return out


def ring_slot_table(w, b: int, through_step: int | None = None) -> np.ndarray:
    """Position held by each slot of sequence b (-1 = empty) after the appends."""
    table = simulate_appends(ring_appended_positions(w, b, through_step), w.sinks, w.window)
    return np.asarray(table, dtype=np.int32)


def paged_expected(w, b: int, step: int, scale=None):
    n = int(w.lengths[b])
    pos = np.arange(n, dtype=np.int64)
    k, v = stored_rows(w, w.rows(TENSOR_K, b, pos).astype(np.float64),
                       w.rows(TENSOR_V, b, pos))
    return attend_heads(w.query(b, step).astype(np.float64), k, v, scale)


def paged_append_expected(w, b: int, step: int, scale=None):
    """Paged workload grown by appends: decode step `step` first appends the
    token at position lengths[b] + step, then attends positions
    0 .. lengths[b] + step (K as given, no RoPE on this workload)."""
    n = int(w.lengths[b]) + step + 1
    pos = np.arange(n, dtype=np.int64)
    k = w.rows(TENSOR_K, b, pos).astype(np.float64)
    v = w.rows(TENSOR_V, b, pos).astype(np.float64)
    return attend_heads(w.query(b, step).astype(np.float64), k, v, scale)


def pool_rows(w, b: int, style: str = "interleaved"):
    """(positions, K rotated + rounded, V) of sequence b's resident tokens."""
    pos = w.resident_positions(b)
    k_raw = w.rows(TENSOR_K, b, pos)
    k, v = stored_rows(w, rope(k_raw, pos[:, None], w.rope_base, style), w.rows(TENSOR_V, b, pos))
    return pos, k, v


def pool_expected(w, b: int, step: int, scale=None, style: str = "interleaved"):
    _, k, v = pool_rows(w, b, style)
    return attend_heads(w.query(b, step).astype(np.float64), k, v, scale)


def pager_schedule(w, b: int):
    """(visible, slots): for each decode step of sequence b, the blocks it
    sees (sorted) and the logical block held by every pool slot (-1 = empty).

    The call order the harness follows: the history streams in (one advance
    per prefill request), step 0's request is met in full, then before
    decode step t the request of step t + 1 is advanced, so step t sees the
    pool with those copies in flight."""
    pool = LruPool(w.pool_slots)
    for r in w.prefill_requests():
        pool.advance(r)
    pool.request(w.step_request(b, 0))
    visible, slots = [], []
    for step in range(w.decode_steps):
        if step + 1 < w.decode_steps:
            pool.advance(w.step_request(b, step + 1))
        visible.append(sorted(pool.visible()))
        slots.append(list(pool.slot_block))
    return visible, slots


def pager_schedule_fused(w, b: int):
    """(visible, slots) as pager_schedule, for the paging step folded into
    the decode (swa_pager_stage of step t + 1's request, then the decode of
    step t, whose launches copy the staged blocks into their slots after the
    attention has read the pool).  Reading: a step attends the blocks
    resident when it starts, i.e. the pool after every earlier copy has
    landed; the staged request's evictions take effect only after that
    attention, so step t still sees the blocks they evict.  `slots` is the
    pool after step t + 1's request is served; every block in it is visible
    once step t's launches are done.  Pinned (tests/test_oracle_paging.py):
    its slot decisions are those of the advance schedule, request for
    request, and a step sees every block the advance schedule shows it."""
    pool = LruPool(w.pool_slots)
    for r in w.prefill_requests():
        pool.advance(r)
    pool.request(w.step_request(b, 0))
    visible, slots = [], []
    for step in range(w.decode_steps):
        pool.commit()
        visible.append(sorted(pool.visible()))
        if step + 1 < w.decode_steps:
            pool.advance(w.step_request(b, step + 1))
        slots.append(list(pool.slot_block))
    return visible, slots


def pager_expected(w, b: int, step: int, blocks, scale=None, style: str = "interleaved"):
    """(out [Hq, d], lse [Hq]) of decode step `step` over the given blocks."""
    blocks = np.asarray(sorted(blocks), dtype=np.int64)
    pos = (blocks[:, None] * w.block_size + np.arange(w.block_size)[None, :]).reshape(-1)
    k_raw = w.rows(TENSOR_K, b, pos)
    v = w.rows(TENSOR_V, b, pos).astype(np.float64)
    k = round_store(rope(k_raw, pos[:, None], w.rope_base, style), w.dtype)
    return attend_heads(w.query(b, step).astype(np.float64), k, v, scale)

"""Counter-based draws of raw Q/K/V rows.

Every row is addressed by (seed, tensor, sequence, position).  Positions are
grouped in chunks of CHUNK consecutive positions; each chunk is drawn from its
own generator seeded with [seed, tensor, sequence, chunk], so the oracle can
regenerate any single position (or any sample of positions) without storing a
whole history, and the GPU harness can generate the same values in bulk.

Values are standard normal (float32) times a scale, then encoded in the
storage dtype: bf16 with round-to-nearest-even, or float32 as drawn.  An
encoded bf16 value is returned as the float32 that holds it exactly.
"""

from __future__ import annotations

import concurrent.futures as _cf
import os

import numpy as np

CHUNK = 64
TENSOR_Q = 0
TENSOR_K = 1
TENSOR_V = 2

# Sequence index reserved for rows that several sequences share (a common
# prompt prefix); kept far above any batch index.
SHARED_SEQUENCE = 1 << 20


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even.

    Finite inputs only (the generators never produce inf/NaN)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    round_bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + round_bias) >> np.uint32(16)).astype(np.uint16)


def f32_from_bf16_bits(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> the float32 values they denote (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def encode_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Encode float32 draws in the storage dtype ("bf16" or "f32")."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return f32_from_bf16_bits(bf16_bits_from_f32(x))
    raise ValueError(f"unknown storage dtype {dtype!r}")


def _draw_chunk(seed: int, tensor: int, seq: int, chunk: int, heads: int, dim: int,
                scale: float) -> np.ndarray:
    gen = np.random.default_rng([int(seed), int(tensor), int(seq), int(chunk)])
    return gen.standard_normal((CHUNK, heads, dim), dtype=np.float32) * np.float32(scale)


def draw_rows(seed: int, tensor: int, seq: int, positions, heads: int, dim: int,
              scale: float, dtype: str) -> np.ndarray:
    """Rows for the given positions of one sequence: float32 [n, heads, dim].

    `positions` is any 1-D collection of non-negative integers (order and
    repeats are kept)."""
    pos = np.asarray(positions, dtype=np.int64).reshape(-1)
    out = np.empty((pos.size, heads, dim), dtype=np.float32)
    if pos.size == 0:
        return out
    if pos.min() < 0:
        raise ValueError("positions must be non-negative")
    chunks = pos // CHUNK
    order = np.argsort(chunks, kind="stable")
    uniq, starts = np.unique(chunks[order], return_index=True)
    bounds = list(starts[1:]) + [pos.size]

    def work(k: int) -> None:
        c = int(uniq[k])
        sel = order[starts[k]:bounds[k]]
        block = _draw_chunk(seed, tensor, seq, c, heads, dim, scale)
        out[sel] = block[pos[sel] - c * CHUNK]

    if uniq.size > 16:
        with _cf.ThreadPoolExecutor(max_workers=_default_workers()) as pool:
            list(pool.map(work, range(uniq.size)))
    else:
        for k in range(uniq.size):
            work(k)
    return encode_storage(out, dtype)


def _default_workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover - non-Linux
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def draw_rows_parallel(seed: int, tensor: int, seq: int, start: int, count: int, heads: int,
                       dim: int, scale: float, dtype: str, workers: int | None = None,
                       out: np.ndarray | None = None) -> np.ndarray:
    """Rows for the contiguous positions [start, start+count) of one sequence.

    Same values as `draw_rows(..., range(start, start+count), ...)`, drawn
    chunk by chunk on a thread pool (numpy releases the GIL while drawing)."""
    if out is None:
        out = np.empty((count, heads, dim), dtype=np.float32)
    if count == 0:
        return out
    first, last = start // CHUNK, (start + count - 1) // CHUNK

    def work(c: int) -> None:
        block = _draw_chunk(seed, tensor, seq, c, heads, dim, scale)
        lo = max(start, c * CHUNK)
        hi = min(start + count, (c + 1) * CHUNK)
        out[lo - start:hi - start] = encode_storage(block[lo - c * CHUNK:hi - c * CHUNK], dtype)

    n = workers or _default_workers()
    if n == 1 or last == first:
        for c in range(first, last + 1):
            work(c)
    else:
        with _cf.ThreadPoolExecutor(max_workers=n) as pool:
            list(pool.map(work, range(first, last + 1)))
    return out

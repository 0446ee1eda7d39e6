"""Loads the synthetic workloads (synth/) into device memory through libswa.

Device memory is allocated with torch; every cache write goes through the
library's own entry points (kv_append_rope for ring caches, kv_write_paged
for pools), so a loaded workload is exactly what the decode path sees in use.
Harness code (not part of the product package), used by the GPU tests, the
smoke check and the benchmark.
"""

from __future__ import annotations

import numpy as np
import torch

from synth import (TENSOR_K, TENSOR_Q, TENSOR_V, PagedAppendWorkload, PagedWorkload,
                   PagerWorkload, PoolWorkload, RingWorkload)
from synth.draws import SHARED_SEQUENCE, draw_rows_parallel

from decode_attention_fixed_amd import binding as B

_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def to_device(arr: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """Upload float32 draws that are exact values of `dtype`."""
    t = torch.from_numpy(np.ascontiguousarray(arr)).to(device, non_blocking=False)
    return t.to(_TORCH_DTYPE[dtype])


class RingState:
    """A ring cache filled with a RingWorkload's history, plus decode buffers."""

    MAX_CALL_TOKENS = 512  # history calls are issued in pieces of at most this many tokens

    def __init__(self, w: RingWorkload, device="cuda", rope_style: str = "interleaved",
                 out_dtype=torch.float32):
        self.w = w
        self.device = device
        self.cache = B.RingCache.allocate(w.batch, w.num_kv_heads, w.head_dim, w.window, w.sinks,
                                          w.cache or w.dtype, w.rope_base, rope_style, device)
        self.workspace = self.cache.workspace(w.num_q_heads)
        self.out = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=out_dtype,
                               device=device)
        self.lse = torch.empty((w.batch, w.num_q_heads), dtype=torch.float32, device=device)

    # -- history -------------------------------------------------------------
    def _rows(self, tensor: int, first: np.ndarray, n: int) -> np.ndarray:
        w = self.w
        heads = w.num_q_heads if tensor == TENSOR_Q else w.num_kv_heads
        out = np.empty((w.batch, n, heads, w.head_dim), dtype=np.float32)
        for b in range(w.batch):
            draw_rows_parallel(w.seed, tensor, b, int(first[b]), n, heads, w.head_dim, w.scale,
                               w.dtype, out=out[b])
        return out

    def append(self, first: np.ndarray, n: int, with_q: bool = False):
        """Appends positions first[b] .. first[b]+n-1 for every sequence in one call;
        returns the rotated query tensor when with_q."""
        k = to_device(self._rows(TENSOR_K, first, n), self.w.dtype, self.device)
        v = to_device(self._rows(TENSOR_V, first, n), self.w.dtype, self.device)
        q = to_device(self._rows(TENSOR_Q, first, n), self.w.dtype, self.device) if with_q else None
        pos = torch.from_numpy(np.asarray(first, dtype=np.int32)).to(self.device)
        B.kv_append_rope(self.cache.handle, k, v, pos, q)
        return q

    def prefill(self, after_call=None) -> None:
        """Issues the workload's history calls (split into pieces of at most
        MAX_CALL_TOKENS tokens, which appends the same tokens in the same order)."""
        for first, n in self.w.history_calls():
            done = 0
            while done < n:
                m = min(self.MAX_CALL_TOKENS, n - done)
                self.append(first + done, m)
                done += m
            if after_call is not None:
                after_call(first, n)

    # -- decode --------------------------------------------------------------
    def step_inputs(self, step: int) -> dict:
        t = self.w.decode_positions(step)
        return dict(
            k=to_device(self._rows(TENSOR_K, t, 1), self.w.dtype, self.device),
            v=to_device(self._rows(TENSOR_V, t, 1), self.w.dtype, self.device),
            q=to_device(self._rows(TENSOR_Q, t, 1), self.w.dtype, self.device),
            pos=torch.from_numpy(t.astype(np.int32)).to(self.device),
        )

    def step(self, inputs: dict, scale: float = 0.0, fused: bool = False) -> None:
        """One decode step.  fused: decode_step_ring (one call; q left as
        given); else kv_append_rope (rotating q in place), then decode_attn_ring."""
        if fused:
            step = (B.decode_step_ring_shifted if self.w.positions == "cache"
                    else B.decode_step_ring)
            step(self.cache.handle, inputs["k"][:, 0], inputs["v"][:, 0], inputs["pos"],
                 inputs["q"][:, 0], self.out, self.workspace, self.lse, scale)
            return
        B.kv_append_rope(self.cache.handle, inputs["k"], inputs["v"], inputs["pos"], inputs["q"])
        B.decode_attn_ring(self.cache.handle, inputs["q"][:, 0], self.out, self.workspace,
                           self.lse, scale)

    def chunk_inputs(self, first_step: int, n: int) -> dict:
        """Raw inputs of decode steps first_step .. first_step + n - 1 as one
        prefill chunk: k, v [B, n, Hkv, d], q [B, n, Hq, d], pos [B]."""
        t = self.w.decode_positions(first_step)
        return dict(
            k=to_device(self._rows(TENSOR_K, t, n), self.w.dtype, self.device),
            v=to_device(self._rows(TENSOR_V, t, n), self.w.dtype, self.device),
            q=to_device(self._rows(TENSOR_Q, t, n), self.w.dtype, self.device),
            pos=torch.from_numpy(t.astype(np.int32)).to(self.device),
        )

    def prefill_chunk(self, inputs: dict, out: torch.Tensor, lse: torch.Tensor | None = None,
                      scale: float = 0.0, workspace: torch.Tensor | None = None) -> None:
        """prefill_attn_ring over one chunk (see chunk_inputs)."""
        w = self.w
        n = inputs["k"].shape[1]
        if workspace is None:
            workspace = B.new_prefill_workspace(w.batch, w.num_q_heads, w.num_kv_heads,
                                                w.head_dim, n, self.device)
        B.prefill_attn_ring(self.cache.handle, inputs["k"], inputs["v"], inputs["pos"],
                            inputs["q"], out, workspace, lse, scale)

    def close(self) -> None:
        self.cache.close()


class PagedState:
    """A paged pool holding a PagedWorkload or a PoolWorkload."""

    def __init__(self, w, device="cuda", out_dtype=torch.float32, rope_style="interleaved"):
        self.w = w
        self.device = device
        if isinstance(w, PagedWorkload):
            table = w.block_table
            self.num_phys = w.num_unique_blocks
            lens = w.lengths
            valid = None
        elif isinstance(w, PoolWorkload):
            table = w.block_table
            self.num_phys = w.batch * w.pool_slots
            lens = np.full(w.batch, w.pool_slots * w.block_size, dtype=np.int64)
            valid = w.block_valid
        else:
            raise TypeError(type(w))
        self.desc = B.make_paged_desc(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                      w.block_size, table.shape[1], self.num_phys,
                                      w.cache or w.dtype)
        self.k_pool, self.v_pool = B.new_pool(self.desc, device)
        self.block_table = torch.from_numpy(np.ascontiguousarray(table, dtype=np.int32)).to(device)
        self.seq_lens = torch.from_numpy(lens.astype(np.int32)).to(device)
        self.block_valid = (torch.from_numpy(np.ascontiguousarray(valid)).to(device)
                            if valid is not None else None)
        self.workspace = B.new_workspace(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                         table.shape[1] * w.block_size, device)
        self.out = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=out_dtype,
                               device=device)
        self.lse = torch.empty((w.batch, w.num_q_heads), dtype=torch.float32, device=device)
        self.rope_style = rope_style

    def _write(self, k: np.ndarray, v: np.ndarray, rows: np.ndarray, pos=None) -> None:
        w = self.w
        if rows.size == 0:
            return
        kd = to_device(k, w.dtype, self.device)
        vd = to_device(v, w.dtype, self.device)
        rd = torch.from_numpy(rows.astype(np.int32)).to(self.device)
        pd = torch.from_numpy(pos.astype(np.int32)).to(self.device) if pos is not None else None
        base = getattr(w, "rope_base", 10000.0)
        B.kv_write_paged(self.desc, self.k_pool, self.v_pool, kd, vd, rd, pd, base,
                         self.rope_style)

    def fill(self) -> None:
        """Writes every resident token's K/V row into its pool row (the physical
        row is block_table[b][i // bs] * bs + i % bs, computed here on the host
        from the workload's table, independently of the kernels)."""
        w = self.w
        bs = w.block_size
        if isinstance(w, PagedWorkload):
            # the shared prefix once, from the shared stream
            pre = w.shared_prefix
            k = draw_rows_parallel(w.seed, TENSOR_K, SHARED_SEQUENCE, 0, pre, w.num_kv_heads,
                                   w.head_dim, w.scale, w.dtype)
            v = draw_rows_parallel(w.seed, TENSOR_V, SHARED_SEQUENCE, 0, pre, w.num_kv_heads,
                                   w.head_dim, w.scale, w.dtype)
            i = np.arange(pre)
            self._write(k, v, w.block_table[0][i // bs].astype(np.int64) * bs + i % bs)
            for b in range(w.batch):
                n = int(w.lengths[b])
                if n <= pre:
                    continue
                k = draw_rows_parallel(w.seed, TENSOR_K, b, pre, n - pre, w.num_kv_heads,
                                       w.head_dim, w.scale, w.dtype)
                v = draw_rows_parallel(w.seed, TENSOR_V, b, pre, n - pre, w.num_kv_heads,
                                       w.head_dim, w.scale, w.dtype)
                i = np.arange(pre, n)
                self._write(k, v, w.block_table[b][i // bs].astype(np.int64) * bs + i % bs)
        else:
            for b in range(w.batch):
                slots = np.nonzero(w.slot_blocks[b] >= 0)[0]
                blocks = w.slot_blocks[b][slots]
                pos = (blocks[:, None] * bs + np.arange(bs)[None, :]).reshape(-1)
                rows = (w.block_table[b][slots].astype(np.int64)[:, None] * bs
                        + np.arange(bs)[None, :]).reshape(-1)
                k = w.rows(TENSOR_K, b, pos)
                v = w.rows(TENSOR_V, b, pos)
                self._write(k, v, rows, pos)

    def step_query(self, step: int) -> torch.Tensor:
        q = np.stack([self.w.query(b, step) for b in range(self.w.batch)])
        return to_device(q, self.w.dtype, self.device)

    def step(self, q: torch.Tensor, scale: float = 0.0) -> None:
        B.decode_attn_paged(self.desc, q, self.k_pool, self.v_pool, self.block_table,
                            self.seq_lens, self.block_valid, self.out, self.workspace, self.lse,
                            scale)


class PagerState:
    """A PagerWorkload: the whole history in pinned host memory, a device pool
    of slots filled on demand by the library's pager, and decode buffers.

    The host store is built with the library's own write path: raw K rows are
    rotated into a device staging pool by kv_write_paged (one block per
    logical block, in order), then copied to the pinned host store."""

    def __init__(self, w: PagerWorkload, device="cuda", out_dtype=torch.float32):
        self.w = w
        self.device = device
        dt = _TORCH_DTYPE[w.dtype]
        B_, L, C = w.batch, w.logical_blocks, w.pool_slots
        blk = (w.num_kv_heads, w.block_size, w.head_dim)
        self.host_k = torch.empty((B_, L) + blk, dtype=dt, pin_memory=True)
        self.host_v = torch.empty((B_, L) + blk, dtype=dt, pin_memory=True)
        self.num_phys = B_ * C
        self.k_pool = torch.zeros((self.num_phys,) + blk, dtype=dt, device=device)
        self.v_pool = torch.zeros((self.num_phys,) + blk, dtype=dt, device=device)
        self.block_table = torch.empty((B_, C), dtype=torch.int32, device=device)
        self.block_valid = torch.empty((B_, C), dtype=torch.uint8, device=device)
        self.seq_lens = torch.full((B_,), C * w.block_size, dtype=torch.int32, device=device)
        self.desc = B.make_paged_desc(B_, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                      w.block_size, C, self.num_phys, w.dtype)
        self.out = torch.empty((B_, w.num_q_heads, w.head_dim), dtype=out_dtype, device=device)
        self.lse = torch.empty((B_, w.num_q_heads), dtype=torch.float32, device=device)
        self.cfg = B.make_pager_config(B_, w.num_kv_heads, w.head_dim, w.block_size, L, C,
                                       self.num_phys, w.dtype)
        self.handle = B.swa_pager_create(self.cfg, self.host_k, self.host_v, self.k_pool,
                                         self.v_pool, w.slot_phys.tolist(), self.block_table,
                                         self.block_valid)
        # the decode's workspace plus the staging area of the folded copies
        self.workspace = torch.empty(B.swa_pager_workspace_bytes(self.handle, w.num_q_heads),
                                     dtype=torch.uint8, device=device)

    def fill_host(self) -> None:
        w = self.w
        bs, L = w.block_size, w.logical_blocks
        n = L * bs
        desc = B.make_paged_desc(1, w.num_kv_heads, w.num_kv_heads, w.head_dim, bs, L, L, w.dtype)
        stage_k = torch.empty((L, w.num_kv_heads, bs, w.head_dim), dtype=self.host_k.dtype,
                              device=self.device)
        stage_v = torch.empty_like(stage_k)
        pos = torch.arange(n, dtype=torch.int32, device=self.device)
        for b in range(w.batch):
            k = draw_rows_parallel(w.seed, TENSOR_K, b, 0, n, w.num_kv_heads, w.head_dim,
                                   w.scale, w.dtype)
            v = draw_rows_parallel(w.seed, TENSOR_V, b, 0, n, w.num_kv_heads, w.head_dim,
                                   w.scale, w.dtype)
            B.kv_write_paged(desc, stage_k, stage_v, to_device(k, w.dtype, self.device),
                             to_device(v, w.dtype, self.device), pos, pos, w.rope_base)
            self.host_k[b].copy_(stage_k.cpu())
            self.host_v[b].copy_(stage_v.cpu())
        torch.cuda.synchronize()

    def reset(self) -> None:
        B.swa_pager_reset(self.handle)

    def advance(self, requests, copy_stream=None) -> int:
        return B.swa_pager_advance(self.handle, requests, None, copy_stream)

    def commit(self) -> None:
        B.swa_pager_commit(self.handle)

    def stage(self, requests) -> int:
        """The next step's requests, copied by the next fused_decode."""
        return B.swa_pager_stage(self.handle, requests)

    def fused_decode(self, q: torch.Tensor, scale: float = 0.0, prepare: bool = False):
        """The decode over the pool, then the staged copies, in its launches."""
        return B.swa_pager_decode(self.handle, self.desc, q, self.k_pool, self.v_pool,
                                  self.block_table, self.seq_lens, self.block_valid, self.out,
                                  self.workspace, self.lse, scale, prepare=prepare)

    def warm(self, copy_stream=None) -> int:
        """The history streams in, then step 0's request is met in full."""
        w = self.w
        n = 0
        for r in w.prefill_requests():
            n += self.advance([r] * w.batch, copy_stream)
        n += self.advance([w.step_request(b, 0) for b in range(w.batch)], copy_stream)
        self.commit()
        return n

    def step_requests(self, step: int) -> list:
        return [self.w.step_request(b, step) for b in range(self.w.batch)]

    def step_query(self, step: int) -> torch.Tensor:
        q = np.stack([self.w.query(b, step) for b in range(self.w.batch)])
        return to_device(q, self.w.dtype, self.device)

    def decode(self, q: torch.Tensor, scale: float = 0.0) -> None:
        B.decode_attn_paged(self.desc, q, self.k_pool, self.v_pool, self.block_table,
                            self.seq_lens, self.block_valid, self.out, self.workspace, self.lse,
                            scale)

    def slot_blocks(self, b: int) -> list:
        return B.swa_pager_slot_blocks(self.handle, b, self.w.pool_slots)

    def close(self) -> None:
        if self.handle:
            torch.cuda.synchronize()
            B.swa_pager_destroy(self.handle)
            self.handle = 0


class BlockPoolState:
    """A paged pool driven by the library's block manager (refcounted blocks,
    prefix sharing, copy-on-write), with the device block table and lengths
    the decode reads, plus decode buffers."""

    def __init__(self, num_blocks: int, block_size: int, max_seqs: int, max_blocks: int,
                 num_q_heads: int, num_kv_heads: int, head_dim: int, dtype: str,
                 device="cuda", out_dtype=torch.float32):
        self.num_blocks, self.block_size = num_blocks, block_size
        self.max_seqs, self.max_blocks = max_seqs, max_blocks
        self.dtype = dtype
        dt = _TORCH_DTYPE[dtype]
        self.handle = B.swa_blocks_create(num_blocks, block_size, max_seqs, max_blocks)
        self.desc = B.make_paged_desc(max_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                      max_blocks, num_blocks, dtype)
        shape = (num_blocks, num_kv_heads, block_size, head_dim)
        self.k_pool = torch.empty(shape, dtype=dt, device=device)
        self.v_pool = torch.empty(shape, dtype=dt, device=device)
        self.block_table = torch.empty((max_seqs, max_blocks), dtype=torch.int32, device=device)
        self.seq_lens = torch.empty((max_seqs,), dtype=torch.int32, device=device)
        B.swa_blocks_sync(self.handle, self.block_table, self.seq_lens)
        self.workspace = B.new_workspace(max_seqs, num_q_heads, num_kv_heads, head_dim,
                                         max_blocks * block_size, device)
        self.out = torch.empty((max_seqs, num_q_heads, head_dim), dtype=out_dtype, device=device)
        self.lse = torch.empty((max_seqs, num_q_heads), dtype=torch.float32, device=device)

    def append(self, seqs, k: torch.Tensor, v: torch.Tensor, rotate: bool = False,
               rope_base: float = 10000.0) -> None:
        B.kv_append_paged(self.handle, self.desc, self.k_pool, self.v_pool, self.block_table,
                          self.seq_lens, seqs, k, v, rotate, rope_base)

    def share(self, src: int, dst: int, n: int) -> None:
        B.swa_blocks_share_prefix(self.handle, src, dst, n, self.block_table, self.seq_lens)

    def free(self, seq: int) -> None:
        B.swa_blocks_free(self.handle, seq, self.seq_lens)

    def state(self) -> dict:
        return B.swa_blocks_state(self.handle, self.max_seqs, self.max_blocks, self.num_blocks)

    def decode(self, q: torch.Tensor, scale: float = 0.0) -> None:
        B.decode_attn_paged(self.desc, q, self.k_pool, self.v_pool, self.block_table,
                            self.seq_lens, None, self.out, self.workspace, self.lse, scale)

    def close(self) -> None:
        if self.handle:
            B.swa_blocks_destroy(self.handle)
            self.handle = 0


def build_paged_append(w: PagedAppendWorkload, extra_steps: int = 0,
                       device="cuda") -> BlockPoolState:
    """The paged workload built through the block manager: the shared prefix
    is appended once to a holder sequence (index B), shared by reference into
    every sequence, the holder is freed (its blocks live on through the
    references), then each sequence's own tokens are appended.  Room is left
    for decode_steps + extra_steps appended tokens per sequence."""
    bs = w.block_size
    steps = w.decode_steps + extra_steps
    lens = [int(x) for x in w.lengths]
    max_blocks = -(-(w.len_range[1] + steps) // bs)
    own = sum(-(-(n + steps) // bs) - min(-(-n // bs), w.shared_blocks) for n in lens)
    num_blocks = w.shared_blocks + own + w.batch
    st = BlockPoolState(num_blocks, bs, w.batch + 1, max_blocks, w.num_q_heads, w.num_kv_heads,
                        w.head_dim, w.dtype, device)
    holder = w.batch
    pre = w.shared_prefix

    def rows(seq, first, n):
        k = draw_rows_parallel(w.seed, TENSOR_K, seq, first, n, w.num_kv_heads, w.head_dim,
                               w.scale, w.dtype)
        v = draw_rows_parallel(w.seed, TENSOR_V, seq, first, n, w.num_kv_heads, w.head_dim,
                               w.scale, w.dtype)
        return (to_device(k, w.dtype, device).unsqueeze(0), to_device(v, w.dtype, device).unsqueeze(0))

    k, v = rows(SHARED_SEQUENCE, 0, pre)
    st.append([holder], k, v)
    for b in range(w.batch):
        st.share(holder, b, min(lens[b], pre))
    st.free(holder)
    for b in range(w.batch):
        if lens[b] > pre:
            k, v = rows(b, pre, lens[b] - pre)
            st.append([b], k, v)
    torch.cuda.synchronize()
    return st

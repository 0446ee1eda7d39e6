#!/usr/bin/env python3
"""Decode-step benchmark on one MI355X.

A step is one pass of the whole decode path over one batch: for the paged /
pool workloads, the decode over the pool and its merge; for the ring
workloads, the RoPE append of the new token and the split-K decode, both done
by one decode_step_ring call (one launch, plus the split merge when a head is
spread over several workgroups; --unfused: kv_append_rope, then
decode_attn_ring).  Inputs are synthetic (synth/), resident in HBM before the
timed region; every step's new-token rows and query are staged on the device
beforehand, and every timed call is marshalled before the timed region (the
timed loops only issue the calls).

The default workload is `paged` (32 sequences of 1K-32K tokens in 16-token
blocks with a 2000-token shared prefix, GQA 32/8, bf16: the largest
configuration and a target of the >= 70 % bar).

Prints one JSON line:
  value            KV-read GB/s of the whole job: algorithmic KV bytes per step
                   (resident rows x Hkv x d x 2 x element bytes, summed over
                   the batch) x steps / time of the timed steps (HIP events
                   at the two ends of the region only).
  roofline         for the dominant kernel (the decode attention kernel, with
                   the small split-merge launch that follows it in the same
                   call when there is one): algorithmic bytes per call / mean
                   call duration, from HIP events recorded on the launch
                   stream at the two ends of a second region of at least 64
                   calls issued back to back, against the 8 TB/s HBM peak;
                   `traffic` is the measured HBM bytes per call from rocprofv3
                   counters (profiles/decode_<workload>_traffic.txt) when they
                   were taken on the current kernel sources, else null.
  cpu_baseline     the float64 NumPy oracle on a bounded sample of the same
                   workload (inputs already in host memory), on the host's
                   cores (the cores this process may run on; the CPU model).
  per_config       the other decode configurations (gqa-ring, long-pool-b1,
                   long-pool-b16, mha-ring), each measured the same way in the
                   same run: steps/s, step GB/s, the decode call's duration,
                   GB/s and fraction of the peak, and the rocprofv3 average of
                   the call's kernels from the committed profile when it was
                   taken on the current kernel sources; then the host-pool
                   paging step (long-pool-swap, with the same decode on the
                   same pool without paging) and the chunked prefill
                   (gqa-prefill: TFLOP/s against the MFMA peak).

Prefill workloads (mha-prefill, gqa-prefill): a step is one prefill_attn_ring
call over a chunk of new tokens per sequence (rotation of the chunk, the
windowed causal attention, the append); `value` and `roofline` are then in
TFLOP/s of useful attention arithmetic (4 x d flops per visible (query head,
key) pair: S = Q K^T and O = P V) against the 2.5 PFLOP/s dense bf16 / fp16
MFMA peak; `roofline` times the whole call (its three launches).

Host-pool paging workload (long-pool-swap): a step is swa_pager_stage for
the next step's block request (LRU decisions on the host) and
swa_pager_decode, whose launches attend the pool as the step found it and
then copy the staged blocks from pinned host memory into the slots they
evict (--pager-mode advance: swa_pager_advance, its copies before the decode,
which does not attend the slots they fill); `value` counts the blocks each
decode actually saw. `swap` reports the blocks and bytes copied per step, and
the same steps without paging on the same pool.

Paged pool grown by appends (paged-append): a step is kv_append_paged of one
token per sequence through the block manager (table and length updates, the
token rows) and the decode over all tokens; KV bytes count each step's
lengths after its append.

--graph issues the timed steps as one captured HIP graph (every step keeps its
own inputs and positions) instead of eager calls; `launch` says which.

Usage: python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                       [--no-per-config] [--graph]
       python bench.py --copy-calibration   (a plain 1 GiB device copy, for counter scaling)
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
PROFILES = os.path.join(ROOT, "profiles")
_CSRC = os.path.join(ROOT, "decode_attention_fixed_amd", "csrc")
DECODE_SRCS = [os.path.join(_CSRC, f) for f in ("decode_mfma.hip", "decode_shared.hip", "decode.hip",
                                                "device_common.h")]
PREFILL_SRCS = [os.path.join(_CSRC, f) for f in ("prefill.hip", "append_rope.hip",
                                                 "device_common.h")]
DEFAULT_WORKLOAD = "paged"
PER_CONFIG = ("gqa-ring", "long-pool-b1", "long-pool-b16", "mha-ring", "long-pool-swap",
              "gqa-prefill")
MIN_CALLS = 64   # decode calls timed back to back for the roofline region


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def describe(w) -> dict:
    if w.kind == "ring":
        what = (f"{w.chunk}-token prefill chunk per sequence per step" if w.chunk
                else "append+decode per step")
        text = (f"{w.name}: B={w.batch}, Hq={w.num_q_heads}, Hkv={w.num_kv_heads}, "
                f"d={w.head_dim}, {w.dtype}, W={w.window} + {w.sinks} sinks, "
                f"history {w.history}, {what}")
        if w.positions == "cache":
            text += ", positions inside the cache (sink position shifting)"
    elif w.kind in ("paged", "paged-append"):
        text = (f"{w.name}: B={w.batch}, Hq={w.num_q_heads}, Hkv={w.num_kv_heads}, "
                f"d={w.head_dim}, {w.dtype}, {w.block_size}-token blocks, lengths "
                f"{w.len_range[0]}..{w.len_range[1]}, shared prefix {w.shared_prefix}")
        if w.kind == "paged-append":
            text += (" shared by reference through the block manager; per step: append one "
                     "token per sequence (kv_append_paged), then decode")
    elif w.kind == "pager":
        text = (f"{w.name}: B={w.batch}, Hq={w.num_q_heads}, Hkv={w.num_kv_heads}, "
                f"d={w.head_dim}, {w.dtype}, {w.logical_blocks} x {w.block_size}-token "
                f"logical blocks in pinned host memory, {w.pool_slots} device slots per "
                f"sequence filled on demand (LRU); per step: {w.window_blocks} window blocks, "
                f"{w.focus_blocks} focus blocks drifting up to {w.focus_drift} per step, "
                f"{w.revisits} random revisits")
    else:
        text = (f"{w.name}: B={w.batch}, Hq={w.num_q_heads}, Hkv={w.num_kv_heads}, "
                f"d={w.head_dim}, {w.dtype}, {w.logical_blocks} x {w.block_size}-token "
                f"logical blocks, pool of {w.pool_slots} slots per sequence")
    if getattr(w, "cache", "") == "i8":
        text += "; int8 cache rows (codes + one float32 scale per row, quantised when written)"
    return {"workload": text, "batch": w.batch, "num_q_heads": w.num_q_heads,
            "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim}


def resident_tokens(w) -> int:
    """Resident rows attended per step, summed over the batch (per kv head)."""
    import numpy as np
    if w.kind == "ring":
        t = w.decode_positions(0)
        return int(sum(min(int(x) + 1, w.slots) for x in t))
    if w.kind == "paged":
        return int(w.lengths.sum())
    return int(np.asarray(w.block_valid, dtype=np.int64).sum()) * w.block_size


def kv_bytes_per_step(w) -> int:
    return resident_tokens(w) * w.kv_bytes_per_token()


def visible_keys(w, t):
    """Keys a query at position t attends on a sink + window ring (t >= 0):
    the last min(t + 1, W) positions, plus the sinks that fall before them."""
    import numpy as np
    t = np.asarray(t, dtype=np.int64)
    return np.minimum(t + 1, w.window) + np.minimum(w.sinks, np.maximum(0, t + 1 - w.window))


def prefill_flops(w, first_positions) -> int:
    """Useful flops of one prefill call whose chunks start at first_positions
    [B]: 2 per multiply-add of S = Q K^T and of O = P V, over visible keys."""
    import numpy as np
    t = np.asarray(first_positions, dtype=np.int64)[:, None] + np.arange(w.chunk)[None, :]
    return int(visible_keys(w, t).sum()) * w.num_q_heads * w.head_dim * 4


def _records(path: str) -> dict:
    rec = {}
    for line in open(path):
        if ":" in line and not line.lstrip().startswith(("#", "|", "-")):
            k, v = line.split(":", 1)
            rec[k.strip()] = v.strip()
    return rec


def traffic_record(name: str, prefix: str = "decode"):
    """Counter-measured HBM bytes per call of workload `name`, if they were
    taken on the current kernel sources."""
    path = os.path.join(PROFILES, f"{prefix}_{name}_traffic.txt")
    if not os.path.exists(path):
        return None
    rec = _records(path)
    if rec.get("source_sha256") != source_sha(prefix):
        return None
    return rec


def profile_call_us(name: str, prefix: str = "decode"):
    """rocprofv3's average duration of one decode call's kernels (attention
    kernel plus merge) from profiles/<prefix>_<name>_kernel_stats.md, if that
    profile was taken on the current kernel sources."""
    path = os.path.join(PROFILES, f"{prefix}_{name}_kernel_stats.md")
    if not os.path.exists(path):
        return None
    rec = _records(path)
    if rec.get("source_sha256") != source_sha(prefix) or "call_us" not in rec:
        return None
    return float(rec["call_us"])


def source_sha(prefix: str = "decode") -> str:
    h = hashlib.sha256()
    for f in (PREFILL_SRCS if prefix == "prefill" else DECODE_SRCS):
        h.update(open(f, "rb").read())
    return h.hexdigest()


def decode_source_sha() -> str:
    return source_sha("decode")


# ---------------------------------------------------------------------------
# GPU side
# ---------------------------------------------------------------------------

class Run:
    """The set-up of one workload on the device: `step[i]` issues timed step i
    (its calls marshalled beforehand), `call[i]` one decode call of the
    roofline region; `close()` frees everything."""

    def __init__(self):
        self.step = []
        self.call = []
        self.closers = []
        self.extra = {}

    def close(self) -> None:
        for c in self.closers:
            c()
        self.step, self.call, self.closers = [], [], []


def setup(w, n_steps: int, n_calls: int, unfused: bool = False,
          pager_mode: str = "fused") -> Run:
    """Stages inputs for n_steps steps and n_calls roofline calls."""
    import numpy as np
    import torch

    from decode_attention_fixed_amd import binding as B
    from tests.device_data import PagedState, RingState, to_device
    from synth import TENSOR_K, TENSOR_Q, TENSOR_V
    from synth.draws import draw_rows_parallel

    run = Run()
    total = n_steps + n_calls
    if w.kind == "ring" and w.chunk:
        # One chunk of rows drawn from the workload, reused by every call at
        # advancing positions (each call rotates and appends it anew).
        st = RingState(w)
        st.prefill()
        inp = st.chunk_inputs(0, w.chunk)
        ws = B.new_prefill_workspace(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                     w.chunk, "cuda")
        out = torch.empty(w.batch, w.chunk, w.num_q_heads, w.head_dim, dtype=torch.bfloat16,
                          device="cuda")
        lse = torch.empty(w.batch, w.chunk, w.num_q_heads, dtype=torch.float32, device="cuda")
        first = w.decode_start[None, :] + w.chunk * np.arange(total)[:, None]
        pos_all = torch.from_numpy(first.astype(np.int32)).cuda()
        calls = [B.prefill_attn_ring(st.cache.handle, inp["k"], inp["v"], pos_all[i], inp["q"],
                                     out, ws, lse, prepare=True) for i in range(total)]
        run.step, run.call = calls[:n_steps], calls[n_steps:]
        run.extra["flops_step"] = [prefill_flops(w, first[i]) for i in range(n_steps)]
        run.extra["flops_call"] = [prefill_flops(w, first[n_steps + i]) for i in range(n_calls)]
        run.closers.append(st.close)
    elif w.kind == "ring":
        st = RingState(w)
        st.prefill()
        start = w.decode_start

        def staged(tensor, heads):
            arr = np.empty((w.batch, total, heads, w.head_dim), dtype=np.float32)
            for b in range(w.batch):
                draw_rows_parallel(w.seed, tensor, b, int(start[b]), total, heads, w.head_dim,
                                   w.scale, w.dtype, out=arr[b])
            t = to_device(arr, w.dtype)                       # [B, total, H, d]
            return t.permute(1, 0, 2, 3).contiguous().unsqueeze(2)  # [total, B, 1, H, d]

        k_all = staged(TENSOR_K, w.num_kv_heads)
        v_all = staged(TENSOR_V, w.num_kv_heads)
        q_all = staged(TENSOR_Q, w.num_q_heads)
        pos_all = torch.from_numpy(
            (start[None, :] + np.arange(total)[:, None]).astype(np.int32)).cuda()
        handle = st.cache.handle
        if unfused:  # the two entry points: append (rotating q in place), then decode
            appends = [B.kv_append_rope(handle, k_all[i], v_all[i], pos_all[i], q_all[i],
                                        prepare=True) for i in range(n_steps)]
            decodes = [B.decode_attn_ring(handle, q_all[i][:, 0], st.out, st.workspace, st.lse,
                                          prepare=True) for i in range(n_steps)]

            def both(a, d):
                def f():
                    a()
                    d()
                return f
            run.step = [both(appends[i], decodes[i]) for i in range(n_steps)]
            # the decode call alone, repeated on the state the last step left
            last = B.decode_attn_ring(handle, q_all[n_steps - 1][:, 0], st.out, st.workspace,
                                      st.lse, prepare=True)
            run.call = [last] * n_calls
        else:  # one call per step: the decode launch appends the token itself
            fn = B.decode_step_ring_shifted if w.positions == "cache" else B.decode_step_ring
            calls = [fn(handle, k_all[i][:, 0], v_all[i][:, 0], pos_all[i], q_all[i][:, 0],
                        st.out, st.workspace, st.lse, prepare=True) for i in range(total)]
            run.step, run.call = calls[:n_steps], calls[n_steps:]
        run.extra["bytes_step"] = run.extra["bytes_call"] = kv_bytes_per_step(w)
        run.closers.append(st.close)
    elif w.kind == "paged-append":
        import ctypes

        from tests.device_data import build_paged_append
        st = build_paged_append(w, extra_steps=total)

        def staged(tensor):
            arr = np.empty((w.batch, n_steps, w.num_kv_heads, w.head_dim), dtype=np.float32)
            for b in range(w.batch):
                draw_rows_parallel(w.seed, tensor, b, int(w.lengths[b]), n_steps, w.num_kv_heads,
                                   w.head_dim, w.scale, w.dtype, out=arr[b])
            t = to_device(arr, w.dtype)                               # [B, steps, Hkv, d]
            return t.permute(1, 0, 2, 3).contiguous().unsqueeze(2)    # [steps, B, 1, Hkv, d]

        k_all, v_all = staged(TENSOR_K), staged(TENSOR_V)
        nq = min(total, w.decode_steps)
        zero = np.zeros((1, w.num_q_heads, w.head_dim), np.float32)
        qs = torch.stack([to_device(np.concatenate([np.stack([w.query(b, i)
                                                              for b in range(w.batch)]), zero]),
                                    w.dtype) for i in range(nq)])
        seqs = (ctypes.c_int32 * w.batch)(*range(w.batch))
        decs = [B.decode_attn_paged(st.desc, qs[j], st.k_pool, st.v_pool, st.block_table,
                                    st.seq_lens, None, st.out, st.workspace, st.lse,
                                    prepare=True) for j in range(nq)]

        def step(i):
            def f():
                st.append(seqs, k_all[i], v_all[i])
                decs[i % nq]()
            return f
        run.step = [step(i) for i in range(n_steps)]
        # the roofline region repeats the decode on the state the steps left
        run.call = [decs[i % nq] for i in range(n_calls)]
        base = int(w.lengths.sum())
        run.extra["bytes_steps"] = [(base + w.batch * (s + 1)) * w.kv_bytes_per_token()
                                    for s in range(n_steps)]
        run.extra["bytes_call"] = (base + w.batch * n_steps) * w.kv_bytes_per_token()
        run.closers.append(st.close)
    elif w.kind == "pager":
        import dataclasses

        from tests.device_data import PagerState
        wl = dataclasses.replace(w, decode_steps=n_steps + 1)
        st = PagerState(wl)
        st.fill_host()
        st.reset()
        copy_stream = torch.cuda.Stream()
        st.warm(copy_stream)
        torch.cuda.synchronize()
        qs = torch.stack([st.step_query(i) for i in range(min(n_steps, w.decode_steps))])
        reqs = [B.pack_requests(st.step_requests(i + 1)) for i in range(n_steps)]
        filled = sum(1 for b in range(w.batch) for x in st.slot_blocks(b) if x >= 0)
        seen, loaded = {}, {}
        host_us = {"advance": 0.0, "decode": 0.0}
        decs = [B.decode_attn_paged(st.desc, qs[j], st.k_pool, st.v_pool, st.block_table,
                                    st.seq_lens, st.block_valid, st.out, st.workspace, st.lse,
                                    prepare=True) for j in range(qs.shape[0])]
        cs = copy_stream if pager_mode == "advance-side-stream" else None

        def advance_step(i):
            # the loads land before the attention: their slots are invalid for it
            def f():
                t = time.perf_counter()
                n = st.advance(reqs[i], cs)
                host_us["advance"] += (time.perf_counter() - t) * 1e6
                loaded[i] = n
                seen[i] = filled - n
                t = time.perf_counter()
                decs[i % len(decs)]()
                host_us["decode"] += (time.perf_counter() - t) * 1e6
            return f

        fused = [st.fused_decode(qs[j], prepare=True) for j in range(qs.shape[0])]

        def fused_step(i):
            # the attention reads the pool as the step found it; the loads
            # for the next step are copied in the same launches, after it
            def f():
                t = time.perf_counter()
                n = st.stage(reqs[i])
                host_us["stage"] += (time.perf_counter() - t) * 1e6
                loaded[i] = n
                seen[i] = filled
                t = time.perf_counter()
                fused[i % len(fused)]()
                host_us["decode"] += (time.perf_counter() - t) * 1e6
            return f
        if pager_mode == "fused":
            # every slot is filled after the warm-up, so each load evicts and
            # the attention of every step sees all of them
            if filled != w.batch * w.pool_slots:
                raise RuntimeError(f"{w.name}: pool not full after the warm-up")
            host_us = {"stage": 0.0, "decode": 0.0}
        step = fused_step if pager_mode == "fused" else advance_step
        run.step = [step(i) for i in range(n_steps)]
        run.extra.update(pager_state=st, pager_seen=seen, pager_loaded=loaded,
                         pager_host_us=host_us, pager_decs=decs, pager_q=qs,
                         block_bytes=2 * w.num_kv_heads * w.block_size * w.head_dim * 2)
        run.closers.append(st.close)
    else:
        st = PagedState(w, out_dtype=torch.float32)
        st.fill()
        qs = torch.stack([st.step_query(i) for i in range(min(total, w.decode_steps))])
        # Pools smaller than the ~256 MB last-level cache are cycled through
        # enough copies (>= 600 MB) that a call cannot be served from cache.
        pool_bytes = st.k_pool.numel() * st.k_pool.element_size() * 2
        copies = max(1, math.ceil(600e6 / pool_bytes)) if pool_bytes < 300e6 else 1
        pools = [(st.k_pool, st.v_pool)] + [(st.k_pool.clone(), st.v_pool.clone())
                                            for _ in range(copies - 1)]
        calls = [B.decode_attn_paged(st.desc, qs[i % qs.shape[0]], *pools[i % copies],
                                     st.block_table, st.seq_lens, st.block_valid, st.out,
                                     st.workspace, st.lse, prepare=True) for i in range(total)]
        run.step, run.call = calls[:n_steps], calls[n_steps:]
        run.extra["bytes_step"] = run.extra["bytes_call"] = kv_bytes_per_step(w)
        run.extra["pool_copies"] = copies

        def free():
            pools.clear()
        run.closers.append(free)
    torch.cuda.synchronize()
    return run


def time_region(fns, graph: bool = False) -> float:
    """ms of issuing every function of `fns` once, in order, between two HIP
    events on the current stream (or one replay of a graph capturing them)."""
    import torch
    begin = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    if graph:
        # captured on the stream the calls were marshalled for (the current one)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=torch.cuda.current_stream()):
            for f in fns:
                f()
        torch.cuda.synchronize()
    torch.cuda.synchronize()
    begin.record()
    if graph:
        g.replay()
    else:
        for f in fns:
            f()
    end.record()
    torch.cuda.synchronize()
    return begin.elapsed_time(end)


def measure(w, steps: int, warmup: int, unfused: bool = False, pager_mode: str = "fused",
            graph: bool = False) -> dict:
    """Sets the workload up and times it, everything on one stream of its own
    (the marshalled calls carry that stream; a graph is captured on it)."""
    import torch
    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        return _measure(w, steps, warmup, unfused, pager_mode, graph)


def _measure(w, steps, warmup, unfused, pager_mode, graph) -> dict:
    import torch
    t0 = time.time()
    # the pager and the block manager keep host state per step: no roofline
    # region of extra steps for them (their region 2 repeats the decode)
    n_calls = 0 if w.kind in ("pager",) else max(steps, MIN_CALLS)
    run = setup(w, warmup + steps, n_calls, unfused, pager_mode)
    log(f"{w.name}: setup {time.time() - t0:.1f} s")
    try:
        for i in range(warmup):
            run.step[i]()
        torch.cuda.synchronize()
        # Region 1: whole steps, events only at the two ends.
        timed = run.step[warmup:warmup + steps]
        wall0 = time.perf_counter()
        total_ms = time_region(timed, graph)
        wall = time.perf_counter() - wall0
        res = {"total_ms": total_ms, "wall_s": wall}
        if w.kind == "pager":
            return _pager_regions(w, run, warmup, steps, res)
        # Region 2: decode calls back to back (the dominant kernel as it runs
        # in a stream), events at the two ends.
        res["calls"] = len(run.call)
        res["decode_ms_mean"] = time_region(run.call) / len(run.call)
        if w.kind == "ring" and w.chunk:
            res["flops_region1"] = sum(run.extra["flops_step"][warmup:])
            res["flops_per_call"] = sum(run.extra["flops_call"]) / len(run.call)
        elif w.kind == "paged-append":
            res["kv_bytes_region1"] = sum(run.extra["bytes_steps"][warmup:])
            res["kv_bytes_call"] = run.extra["bytes_call"]
        else:
            res["kv_bytes_region1"] = run.extra["bytes_step"] * steps
            res["kv_bytes_call"] = run.extra["bytes_call"]
        return res
    finally:
        run.close()
        torch.cuda.synchronize()
        torch.cuda.empty_cache()


def _pager_regions(w, run, warmup, steps, res) -> dict:
    import torch

    from decode_attention_fixed_amd import binding as B
    st = run.extra["pager_state"]
    timed = range(warmup, warmup + steps)
    res["host_us_per_step"] = {k: round(v / (warmup + steps), 1)
                               for k, v in run.extra["pager_host_us"].items()}
    res["kv_bytes_region1"] = sum(run.extra["pager_seen"][i] for i in timed) * w.block_size * \
        w.kv_bytes_per_token()
    res["blocks_loaded_region1"] = sum(run.extra["pager_loaded"][i] for i in timed)
    res["block_bytes"] = run.extra["block_bytes"]
    st.commit()
    torch.cuda.synchronize()
    # Region 2: the decode alone, back to back, over cycled copies of the pool
    # (>= 600 MB together, so none is served from the last-level cache).
    pool_bytes = st.k_pool.numel() * st.k_pool.element_size() * 2
    copies = max(1, math.ceil(600e6 / pool_bytes))
    pools = [(st.k_pool, st.v_pool)] + [(st.k_pool.clone(), st.v_pool.clone())
                                        for _ in range(copies - 1)]
    visible = int(st.block_valid.sum().item())
    decs = run.extra["pager_decs"]
    q0 = run.extra["pager_q"][0]
    cyc = [B.decode_attn_paged(st.desc, q0, k, v, st.block_table, st.seq_lens, st.block_valid,
                               st.out, st.workspace, st.lse, prepare=True) for k, v in pools]
    n = max(steps, MIN_CALLS)
    for i in range(warmup):
        cyc[i % copies]()
    res["calls"] = n
    res["decode_ms_mean"] = time_region([cyc[s % copies] for s in range(n)]) / n
    res["kv_bytes_call"] = visible * w.block_size * w.kv_bytes_per_token()
    # Region 3: the same steps without paging, on the one live pool (the
    # cache conditions of region 1): what the paging adds to a step.
    res["no_swap_ms"] = time_region([decs[s % len(decs)] for s in range(steps)]) / steps
    pools.clear()
    return res


# ---------------------------------------------------------------------------
# CPU oracle baseline
# ---------------------------------------------------------------------------

def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(w, budget_s: float = 15.0) -> dict:
    """Times the float64 oracle on whole (sequence, decode step) samples, in
    step order, until `budget_s` seconds of oracle arithmetic are timed; the
    inputs of each sample are drawn beforehand (host memory) and only the
    oracle's arithmetic is timed."""
    import numpy as np
    import threadpoolctl

    from oracle.attention import attend_heads
    from oracle.decode import stored_rows
    from oracle.ring import resident_positions
    from oracle.rope import rope
    from oracle.rounding import round_store
    from synth import TENSOR_K, TENSOR_Q, TENSOR_V

    def inputs(b, step):
        if w.kind == "ring":
            t = int(w.decode_positions(step)[b])
            pos = np.asarray(resident_positions(t, w.sinks, w.window))
            return (pos, t, w.rows(TENSOR_K, b, pos), w.rows(TENSOR_V, b, pos),
                    w.rows(TENSOR_Q, b, [t])[0])
        if w.kind == "paged":
            pos = np.arange(int(w.lengths[b]))
            return pos, None, w.rows(TENSOR_K, b, pos), w.rows(TENSOR_V, b, pos), w.query(b, step)
        if w.kind == "paged-append":
            pos = np.arange(int(w.lengths[b]) + step + 1)
            return pos, None, w.rows(TENSOR_K, b, pos), w.rows(TENSOR_V, b, pos), w.query(b, step)
        if w.kind == "pager":
            blocks = np.asarray(pager_sets[b][step], dtype=np.int64)
            pos = (blocks[:, None] * w.block_size + np.arange(w.block_size)[None, :]).reshape(-1)
            return pos, None, w.rows(TENSOR_K, b, pos), w.rows(TENSOR_V, b, pos), w.query(b, step)
        pos = w.resident_positions(b)
        return pos, None, w.rows(TENSOR_K, b, pos), w.rows(TENSOR_V, b, pos), w.query(b, step)

    if w.kind == "pager":
        from oracle.decode import pager_schedule
        pager_sets = [pager_schedule(w, b)[0] for b in range(w.batch)]

    def oracle_step(pos, t, k_raw, v, q_raw):
        if w.kind == "ring" and getattr(w, "positions", "") == "cache":
            c = np.arange(len(pos))  # cache indices: the resident positions in order
            k = rope(k_raw, c[:, None], w.rope_base)
            q = rope(q_raw, len(pos) - 1, w.rope_base)
            v = np.asarray(v, dtype=np.float64)
        elif w.kind == "ring":
            k, v = stored_rows(w, rope(k_raw, pos[:, None], w.rope_base), v)
            q = round_store(rope(q_raw, t, w.rope_base), w.dtype)
        elif w.kind in ("paged", "paged-append"):
            k, v = stored_rows(w, k_raw.astype(np.float64), v)
            q = q_raw.astype(np.float64)
        else:
            k, v = stored_rows(w, rope(k_raw, pos[:, None], w.rope_base), v)
            q = q_raw.astype(np.float64)
        return attend_heads(q, k, v)

    oracle_step(*inputs(0, 0))  # untimed: first-touch of the arrays and BLAS start-up
    timed, n, step, done, flops = 0.0, 0, 0, False, 0
    while not done:
        for b in range(w.batch):
            args = inputs(b, step)
            t0 = time.perf_counter()
            oracle_step(*args)
            timed += time.perf_counter() - t0
            n += 1
            if w.kind == "ring" and w.chunk:
                flops += int(visible_keys(w, args[1])) * w.num_q_heads * w.head_dim * 4
            if timed >= budget_s:
                done = True
                break
        step += 1
        done = done or step >= w.decode_steps
    per_seq = timed / n
    steps_per_s = 1.0 / (per_seq * w.batch)
    blas = max([p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()] or [1])
    cores = len(os.sched_getaffinity(0))
    host = {"cores": cores, "blas_threads": blas, "cpu_model": cpu_model(), "kind": "oracle"}
    if w.kind == "ring" and w.chunk:
        return {"value": round(flops / timed / 1e12, 6), "unit": "TFLOP/s", **host,
                "sample": (f"{n} (sequence, chunk row) samples of {w.name} (sequences in "
                           f"order, rows from the first chunk's first; all heads; a chunk "
                           f"row is the decode step at its position), inputs pre-drawn in "
                           f"host memory; float64 NumPy, {timed:.1f} s timed; {cores} cores "
                           f"available, BLAS threads {blas}, elementwise ops on one thread; "
                           f"useful flops of the sampled rows / time")}
    if w.kind == "pager":
        step_bytes = len(pager_sets[0][0]) * w.block_size * w.kv_bytes_per_token() * w.batch
    elif w.kind == "paged-append":
        step_bytes = (int(w.lengths.sum()) + w.batch) * w.kv_bytes_per_token()
    else:
        step_bytes = kv_bytes_per_step(w)
    return {"value": round(steps_per_s * step_bytes / 1e9, 4), "unit": "GB/s",
            "steps_per_s": round(steps_per_s, 4), **host,
            "sample": (f"{n} (sequence, decode step) samples of {w.name} (sequences in order, "
                       f"steps from 0; all heads), inputs pre-drawn in host memory; float64 "
                       f"NumPy, {timed:.1f} s timed; {cores} cores available, BLAS threads "
                       f"{blas}, elementwise ops on one thread; scaled to one step of the "
                       f"full batch")}


def copy_calibration(nbytes: int = 1 << 30) -> None:
    """A plain device-to-device copy of known size: its FETCH_SIZE / WRITE_SIZE
    counter readings scale the decode kernel's readings to bytes."""
    import torch
    torch.cuda.set_device(0)
    x = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(5):
        y.copy_(x)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / 5
    print(json.dumps({"copy_bytes": nbytes, "ms": round(ms, 4),
                      "gbs_read_plus_write": round(2 * nbytes / ms / 1e6, 1)}), flush=True)


def copy_engine_probe(block_bytes: int = 64 << 10, blocks: int = 256, reps: int = 4) -> dict:
    """What one host-to-device copy through the copy engine costs: `blocks`
    scattered blocks of `block_bytes` from pinned host memory, one
    hipMemcpyAsync each (torch's non-blocking copy_), against one copy of the
    same bytes contiguous.  The pager moves its blocks with a kernel instead
    (one launch for all of a step's blocks)."""
    import numpy as np
    import torch
    torch.cuda.set_device(0)
    n = block_bytes // 2
    src = torch.empty((blocks, n), dtype=torch.int16, pin_memory=True).fill_(1)
    dst = torch.empty((blocks, n), dtype=torch.int16, device="cuda")
    order = np.random.default_rng(0).permutation(blocks)
    stream = torch.cuda.Stream()
    out = {}
    with torch.cuda.stream(stream):
        for kind in ("per_block", "contiguous"):
            def run():
                if kind == "per_block":
                    for i in order:
                        dst[int(i)].copy_(src[int(i)], non_blocking=True)
                else:
                    dst.copy_(src, non_blocking=True)
            run()
            stream.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0 = time.perf_counter()
            a.record(stream)
            for _ in range(reps):
                run()
            b.record(stream)
            b.synchronize()
            wall = (time.perf_counter() - t0) * 1e3 / reps
            ms = a.elapsed_time(b) / reps
            calls = blocks if kind == "per_block" else 1
            out[kind] = {"copies": calls, "bytes_each": block_bytes * blocks // calls,
                         "gpu_us_per_copy": round(ms * 1e3 / calls, 2),
                         "host_us_per_copy": round(wall * 1e3 / calls, 2),
                         "gbs": round(block_bytes * blocks / ms / 1e6, 2)}
    return {"copy_engine_probe": out}


def read_ceiling(nbytes: int = 4 << 30, reps: int = 20) -> dict:
    """The HBM read rate the chip achieves: swa_stream_read (nontemporal
    16-byte loads, 2048 workgroups, nothing written but one word per wave)
    over a buffer far larger than the caches, timed with HIP events on its
    own stream."""
    import torch
    from decode_attention_fixed_amd import binding as B
    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        x = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
        sink = torch.empty(B.STREAM_READ_SINK_BYTES, dtype=torch.uint8, device="cuda")
        for _ in range(3):
            B.stream_read(x, sink, stream)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            B.stream_read(x, sink, stream)
        b.record(stream)
        b.synchronize()
        ms = a.elapsed_time(b) / reps
    del x, sink
    torch.cuda.empty_cache()
    return {"read_gbs": round(nbytes / ms / 1e6, 1), "bytes": nbytes, "reps": reps,
            "kernel": "swa_stream_read"}


# ---------------------------------------------------------------------------
# the JSON line
# ---------------------------------------------------------------------------

def prefill_line(w, args, res) -> dict:
    ms_per_step = res["total_ms"] / args.steps
    value = res["flops_region1"] / (res["total_ms"] / 1e3) / 1e12
    per_call = res["flops_per_call"]
    achieved = per_call / (res["decode_ms_mean"] / 1e3) / 1e12
    traffic = traffic_record(w.name, "prefill")
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": (int(float(traffic["fetch_bytes_per_call"])
                                + float(traffic["write_bytes_per_call"]))
                            if traffic else None),
                "kernel": ("prefill call: chunk rotation, the windowed causal attention "
                           "kernel (S in bf16, P V in fp16 MFMA, fp32 accumulation) and the "
                           "append, on the launch stream, timed together"),
                "calls": res["calls"], "call_us": round(res["decode_ms_mean"] * 1e3, 2),
                "algorithmic_flops": int(per_call)}
    return {
        "metric": "prefill-attention TFLOP/s", "value": round(value, 2), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic", "config": describe(w),
        "tokens_per_s": round(w.batch * w.chunk * 1e3 / ms_per_step, 1),
        "roofline": roofline,
        "launch": "one HIP graph of the timed steps" if args.graph else "eager calls",
    }


def decode_numbers(w, steps: int, res: dict) -> dict:
    ms_per_step = res["total_ms"] / steps
    value = res["kv_bytes_region1"] / (res["total_ms"] / 1e3) / 1e9
    achieved = res["kv_bytes_call"] / (res["decode_ms_mean"] / 1e3) / 1e9
    return {"ms_per_step": ms_per_step, "value": value, "achieved": achieved,
            "call_us": res["decode_ms_mean"] * 1e3}


def per_config_entry(name: str, args, ceiling_gbs: float | None = None) -> dict:
    from synth import WORKLOADS
    w = WORKLOADS[name]
    res = measure(w, args.steps, args.warmup)
    if w.kind == "ring" and w.chunk:  # chunked prefill: flops against the MFMA peak
        line = prefill_line(w, args, res)
        r = line["roofline"]
        prof = profile_call_us(name, "prefill")
        return {"workload": line["config"]["workload"], "tokens_per_s": line["tokens_per_s"],
                "ms_per_step": line["ms_per_step"], "tflops": line["value"],
                "call_us": r["call_us"], "call_tflops": r["achieved"], "bound": "mfma",
                "frac": r["frac"], "profile_call_us": prof,
                "algorithmic_flops": r["algorithmic_flops"]}
    n = decode_numbers(w, args.steps, res)
    prof = profile_call_us(name)
    extra = {}
    if w.kind == "pager":
        extra["swap"] = {"mode": "fused",
                         "blocks_per_step": round(res["blocks_loaded_region1"] / args.steps, 3),
                         "no_swap_ms_per_step": round(res["no_swap_ms"], 5)}
    return {"workload": describe(w)["workload"],
            "steps_per_s": round(1e3 / n["ms_per_step"], 1),
            "ms_per_step": round(n["ms_per_step"], 5), "gbs": round(n["value"], 1),
            "call_us": round(n["call_us"], 2), "call_gbs": round(n["achieved"], 1),
            "frac": round(n["achieved"] / HBM_PEAK_GBS, 4),
            "frac_of_read_ceiling": (round(n["achieved"] / ceiling_gbs, 4)
                                     if ceiling_gbs else None),
            "profile_call_us": prof,
            "profile_frac": (round(res["kv_bytes_call"] / (prof * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
                             if prof else None),
            "algorithmic_bytes": res["kv_bytes_call"], **extra}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-per-config", action="store_true",
                    help="measure the named workload only (the profiling runs use this)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--copy-engine-probe", action="store_true",
                    help="print only the cost of host-to-device block copies through the copy "
                         "engine (one hipMemcpyAsync per 64 KiB block, and one contiguous copy)")
    ap.add_argument("--read-ceiling", action="store_true",
                    help="print only the streaming HBM read rate (swa_stream_read)")
    ap.add_argument("--no-read-ceiling", action="store_true")
    ap.add_argument("--unfused", action="store_true",
                    help="ring caches: kv_append_rope + decode_attn_ring per step instead of "
                         "decode_step_ring")
    ap.add_argument("--graph", action="store_true",
                    help="issue the timed steps as one captured HIP graph (ring caches and "
                         "read-only pools; the pager and the block manager run host logic "
                         "every step)")
    ap.add_argument("--pager-mode", choices=("fused", "advance", "advance-side-stream"),
                    default="fused",
                    help="long-pool-swap: 'fused' stages the next step's loads and copies "
                         "them in the decode's own launches, after the attention read the "
                         "pool (swa_pager_stage + swa_pager_decode); 'advance' copies them "
                         "before the decode on the attention stream (swa_pager_advance); "
                         "'advance-side-stream' does so on a stream of its own")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures the decode path on one GPU only; --gpus {args.gpus} "
              f"(WORLD_SIZE {world}) is not supported: run with --gpus 1", file=sys.stderr)
        return 2

    if args.copy_calibration:
        copy_calibration()
        return 0
    if args.copy_engine_probe:
        print(json.dumps(copy_engine_probe()), flush=True)
        return 0
    if args.read_ceiling:
        print(json.dumps(read_ceiling()), flush=True)
        return 0

    from synth import WORKLOADS
    w = WORKLOADS[args.workload]
    if args.graph and w.kind in ("pager", "paged-append"):
        print(f"--graph: workload {w.name} runs host logic every step and is not captured",
              file=sys.stderr)
        return 2
    res = measure(w, args.steps, args.warmup, args.unfused, args.pager_mode, args.graph)
    if w.kind == "ring" and w.chunk:
        out = prefill_line(w, args, res)
        if not args.no_cpu_baseline:
            out["cpu_baseline"] = cpu_baseline(w)
        print(json.dumps(out), flush=True)
        return 0
    n = decode_numbers(w, args.steps, res)
    traffic = traffic_record(w.name)
    prof = profile_call_us(w.name)
    roofline = {"bound": "hbm", "achieved": round(n["achieved"], 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(n["achieved"] / HBM_PEAK_GBS, 4),
                "traffic": (int(float(traffic["fetch_bytes_per_call"])
                                + float(traffic["write_bytes_per_call"]))
                            if traffic else None),
                "kernel": ("decode call: the attention kernel, plus the split merge "
                           "launch when a head's rows are spread over several workgroups; "
                           "both on the launch stream, timed together"),
                "calls": res["calls"], "call_us": round(n["call_us"], 2),
                "profile_call_us": prof,
                "algorithmic_bytes": res["kv_bytes_call"]}
    out = {
        "metric": "decode-attention KV-read GB/s", "value": round(n["value"], 1), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(n["ms_per_step"], 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8" if getattr(w, "cache", "") == "i8" else ("bf16" if w.dtype == "bf16" else "f32"),
        "data": "synthetic", "config": describe(w),
        "steps_per_s": round(1e3 / n["ms_per_step"], 1),
        "hbm_frac_of_peak": round(n["value"] / HBM_PEAK_GBS, 4),
        "roofline": roofline,
        "launch": "one HIP graph of the timed steps" if args.graph else "eager calls",
    }
    if w.kind == "pager":
        per_step = res["blocks_loaded_region1"] / args.steps
        out["swap"] = {
            "blocks_per_step": round(per_step, 3),
            "bytes_per_step": int(per_step * res["block_bytes"]),
            "host_to_device_gbs": round(per_step * res["block_bytes"] / n["ms_per_step"] / 1e6, 2),
            "no_swap_ms_per_step": round(res["no_swap_ms"], 5),
            "host_us_per_step": res["host_us_per_step"],
            "wall_ms_per_step": round(res["wall_s"] * 1e3 / args.steps, 5),
            "mode": args.pager_mode,
            "copies_on": {"fused": "extra workgroups of the decode's merge launch",
                          "advance": "a launch of their own before the decode, on the "
                                     "attention stream",
                          "advance-side-stream": "a launch of their own on a stream of "
                                                 "its own"}[args.pager_mode],
            "note": ("copies from pinned host memory; no_swap_ms_per_step is the same "
                     "decode on the same pool without paging"),
        }
    ceiling = None
    if not args.no_read_ceiling:
        ceiling = read_ceiling()
        roofline["read_ceiling_gbs"] = ceiling["read_gbs"]
        roofline["frac_of_read_ceiling"] = round(n["achieved"] / ceiling["read_gbs"], 4)
        log(f"streaming read ceiling {ceiling['read_gbs']} GB/s")
    if not args.no_per_config and w.name == DEFAULT_WORKLOAD and not args.graph:
        out["per_config"] = []
        for name in PER_CONFIG:
            out["per_config"].append(per_config_entry(name, args,
                                                      ceiling["read_gbs"] if ceiling else None))
            e = out["per_config"][-1]
            log(f"per-config {name}: " + (f"{e['call_gbs']} GB/s per call" if "call_gbs" in e
                                          else f"{e['call_tflops']} TFLOP/s per call"))
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

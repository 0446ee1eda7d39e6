"""The C-ABI used from plain C, with no Python or PyTorch in the process.

tests/capi/capi_check.c (built by __graft_entry__.build() with gcc against
include/swa.h, the HIP runtime's C API and the in-tree libswa.so) allocates
a ring cache with hipMalloc, appends a history with kv_append_rope, and runs
fused decode steps with decode_step_ring; with --pool it fills a NaN-poisoned
paged pool (bf16, or int8 codes quantised by the write) with kv_write_paged
(K rotated on the way in) and runs
decode_attn_paged over a block table with absent slots.  Its inputs are the
seeded synthetic rows, written to a file here; its outputs are checked
against the float64 oracle with the usual bars (slot table exact, outputs
within 2e-3, lse within 1e-3).
"""

import os
import subprocess

import numpy as np
import pytest
import torch

from oracle.decode import pool_expected, ring_expected, ring_slot_table
from synth import TENSOR_K, TENSOR_Q, TENSOR_V, PoolWorkload, RingWorkload

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BIN = os.path.join(ROOT, "tests", "capi", "capi_check")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _bf16_bytes(a: np.ndarray) -> bytes:
    """float32 values that are exact bf16 numbers -> their bf16 bytes."""
    bits = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    assert np.all((bits & 0xFFFF) == 0)
    return (bits >> 16).astype(np.uint16).tobytes()


@pytest.mark.parametrize("kw", [
    dict(),                                                        # g = 4, wrapped ring
    dict(num_q_heads=4, num_kv_heads=4, seed=73, history="prefill:40", rope_style=1),  # g = 1
])
def test_capi_ring_steps(tmp_path, kw):
    assert os.path.exists(BIN), f"{BIN} is not built: run __graft_entry__.build()"
    kw = dict(kw)
    rope_half = kw.pop("rope_style", 0)
    base = dict(name="capi", seed=71, batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128,
                dtype="bf16", window=200, sinks=4, rope_base=10000.0, scale=0.5,
                decode_steps=4, history="prefill:300")
    base.update(kw)
    w = RingWorkload(**base)
    (first, n_hist), = w.history_calls()
    B, hq, hkv, d, n = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.decode_steps

    hist = [np.stack([w.rows(t, b, np.arange(first[b], first[b] + n_hist)) for b in range(B)])
            for t in (TENSOR_K, TENSOR_V)]                                    # [B, n_hist, Hkv, d]
    pos = np.stack([w.decode_positions(s) for s in range(n)]).astype(np.int32)  # [n, B]
    steps = {t: np.stack([np.stack([w.rows(t, b, pos[s, b:b + 1])[0] for b in range(B)])
                          for s in range(n)]) for t in (TENSOR_K, TENSOR_V, TENSOR_Q)}

    inp = tmp_path / "in.bin"
    out = tmp_path / "out.bin"
    with open(inp, "wb") as f:
        f.write(np.array([B, hq, hkv, d, w.window, w.sinks, n_hist, n, rope_half],
                         dtype=np.int32).tobytes())
        f.write(np.array([w.rope_base], dtype=np.float32).tobytes())
        f.write(_bf16_bytes(hist[0]))
        f.write(_bf16_bytes(hist[1]))
        f.write(_bf16_bytes(steps[TENSOR_K]))
        f.write(_bf16_bytes(steps[TENSOR_V]))
        f.write(_bf16_bytes(steps[TENSOR_Q]))
        f.write(first.astype(np.int32).tobytes())
        f.write(pos.tobytes())
    print(f"capi_check {kw}", flush=True)
    res = subprocess.run([BIN, str(inp), str(out)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr

    raw = np.fromfile(out, dtype=np.uint8)
    n_out, n_lse = n * B * hq * d, n * B * hq
    got = raw[:4 * n_out].view(np.float32).reshape(n, B, hq, d)
    lse = raw[4 * n_out:4 * (n_out + n_lse)].view(np.float32).reshape(n, B, hq)
    sp = raw[4 * (n_out + n_lse):].view(np.int32).reshape(B, w.sinks + w.window)
    style = "half" if rope_half else "interleaved"
    for s in range(n):
        for b in range(B):
            want, want_lse = ring_expected(w, b, s, style=style)
            assert float(np.abs(got[s, b] - want).max()) <= 2e-3, (s, b)
            assert float(np.abs(lse[s, b] - want_lse).max()) <= 1e-3, (s, b)
    for b in range(B):
        assert np.array_equal(sp[b], ring_slot_table(w, b, n - 1)), b
    print(style, res.stdout.strip(), flush=True)


@pytest.mark.parametrize("seed,rope_half,cache", [(61, 0, ""), (69, 1, ""), (66, 0, "i8")])
def test_capi_pool_steps(tmp_path, seed, rope_half, cache):
    assert os.path.exists(BIN), f"{BIN} is not built: run __graft_entry__.build()"
    w = PoolWorkload(name="capi-pool", seed=seed, batch=3, num_q_heads=6, num_kv_heads=2,
                     head_dim=128, dtype="bf16", block_size=32, logical_blocks=48,
                     pool_slots=16, rope_base=10000.0, scale=0.5, decode_steps=3, cache=cache)
    B, hq, hkv, d, n, bs = (w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim,
                            w.decode_steps, w.block_size)
    valid = w.block_valid
    assert valid.min() == 0  # some slots absent: their poisoned rows must stay unread
    ks, vs, rows, pos = [], [], [], []
    for b in range(B):  # every resident block of b, rows named from its table entry
        slots = np.nonzero(w.slot_blocks[b] >= 0)[0]
        p = (w.slot_blocks[b][slots][:, None] * bs + np.arange(bs)[None, :]).reshape(-1)
        r = (w.block_table[b][slots].astype(np.int64)[:, None] * bs
             + np.arange(bs)[None, :]).reshape(-1)
        ks.append(w.rows(TENSOR_K, b, p))
        vs.append(w.rows(TENSOR_V, b, p))
        rows.append(r)
        pos.append(p)
    ks, vs = np.concatenate(ks), np.concatenate(vs)
    rows, pos = np.concatenate(rows), np.concatenate(pos)
    q = np.stack([np.stack([w.query(b, s) for b in range(B)]) for s in range(n)])
    lens = np.full(B, w.pool_slots * bs, dtype=np.int32)

    inp = tmp_path / "in.bin"
    out = tmp_path / "out.bin"
    with open(inp, "wb") as f:
        f.write(np.array([B, hq, hkv, d, bs, w.pool_slots, B * w.pool_slots, len(rows), n,
                          rope_half, int(cache == "i8")], dtype=np.int32).tobytes())
        f.write(np.array([w.rope_base], dtype=np.float32).tobytes())
        f.write(_bf16_bytes(ks))
        f.write(_bf16_bytes(vs))
        f.write(rows.astype(np.int32).tobytes())
        f.write(pos.astype(np.int32).tobytes())
        f.write(np.ascontiguousarray(w.block_table, dtype=np.int32).tobytes())
        f.write(lens.tobytes())
        f.write(np.ascontiguousarray(valid, dtype=np.uint8).tobytes())
        f.write(_bf16_bytes(q))
    print(f"capi_check --pool seed={seed} rope_half={rope_half} cache={cache!r}", flush=True)
    res = subprocess.run([BIN, "--pool", str(inp), str(out)], capture_output=True, text=True,
                         timeout=120)
    assert res.returncode == 0, res.stderr

    raw = np.fromfile(out, dtype=np.float32)
    got = raw[:n * B * hq * d].reshape(n, B, hq, d)
    lse = raw[n * B * hq * d:].reshape(n, B, hq)
    style = "half" if rope_half else "interleaved"
    for s in range(n):
        for b in range(B):
            want, want_lse = pool_expected(w, b, s, style=style)
            assert float(np.abs(got[s, b] - want).max()) <= 2e-3, (s, b)
            assert float(np.abs(lse[s, b] - want_lse).max()) <= 1e-3, (s, b)
    print(res.stdout.strip(), flush=True)

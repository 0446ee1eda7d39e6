"""The input generators: determinism, counter addressing, encodings and the
structure of the workloads (lengths, shared prefix, block tables, residency)."""

import numpy as np
import torch

from synth import (TENSOR_K, TENSOR_V, WORKLOADS, bf16_bits_from_f32, draw_rows,
                   draw_rows_parallel, f32_from_bf16_bits)


def test_rows_are_addressed_by_position_only():
    a = draw_rows(7, TENSOR_K, 3, range(0, 200), 2, 16, 0.5, "bf16")
    b = draw_rows(7, TENSOR_K, 3, [150, 3, 64, 63], 2, 16, 0.5, "bf16")
    assert np.array_equal(b, a[[150, 3, 64, 63]])
    c = draw_rows_parallel(7, TENSOR_K, 3, 37, 150, 2, 16, 0.5, "bf16", workers=4)
    assert np.array_equal(c, a[37:187])


def test_streams_differ():
    a = draw_rows(7, TENSOR_K, 3, range(64), 2, 16, 1.0, "f32")
    assert not np.array_equal(a, draw_rows(7, TENSOR_V, 3, range(64), 2, 16, 1.0, "f32"))
    assert not np.array_equal(a, draw_rows(7, TENSOR_K, 4, range(64), 2, 16, 1.0, "f32"))
    assert not np.array_equal(a, draw_rows(8, TENSOR_K, 3, range(64), 2, 16, 1.0, "f32"))


def test_bf16_encoding_is_round_to_nearest_even():
    x = np.random.default_rng(0).standard_normal(50_000).astype(np.float32)
    got = f32_from_bf16_bits(bf16_bits_from_f32(x))
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(got, want)


def test_distribution():
    x = draw_rows(1, TENSOR_K, 0, range(4096), 4, 32, 0.5, "f32")
    assert abs(x.mean()) < 0.01 and abs(x.std() - 0.5) < 0.01


def test_ring_workloads():
    w = WORKLOADS["mha-ring"]
    calls = w.history_calls()
    assert len(calls) == 32 and all(n == 256 for _, n in calls)
    assert int(w.decode_start[0]) == 8192
    g = WORKLOADS["gqa-ring"]
    st = g.decode_start
    assert st.shape == (64,) and st.min() >= 4096 and st.max() < 65536
    (p0, n0), (p1, n1) = g.history_calls()
    assert n0 == 4 and np.all(p0 == 0) and n1 == 4096 and np.all(p1 == st - 4096)
    t = WORKLOADS["tiny-ring"]
    assert t.history_calls()[0][1] == 20 and int(t.decode_start[0]) == 20


def test_paged_workload_structure():
    w = WORKLOADS["paged"]
    L = w.lengths
    assert L.min() >= 1024 and L.max() <= 32768 and L.shape == (32,)
    bt = w.block_table
    assert bt.shape == (32, 2048)
    used = []
    for b in range(32):
        nb = -(-int(L[b]) // 16)
        assert np.all(bt[b, nb:] == -1) and np.all(bt[b, :nb] >= 0)
        # the shared prefix (2000 tokens = 125 blocks) maps to the same physical ids
        assert np.array_equal(bt[b, :min(nb, 125)], bt[0, :min(nb, 125)])
        used.append(bt[b, min(nb, 125):nb])
    priv = np.concatenate(used)
    assert len(np.unique(priv)) == priv.size                  # private blocks are unique
    allids = np.concatenate([bt[0, :125], priv])
    assert np.array_equal(np.sort(allids), np.arange(w.num_unique_blocks))
    # shared rows are the same draw for every sequence, private rows differ
    a = w.rows(TENSOR_K, 0, [5, 1999, 2000])
    b = w.rows(TENSOR_K, 9, [5, 1999, 2000])
    assert np.array_equal(a[:2], b[:2]) and not np.array_equal(a[2], b[2])


def test_pool_workload_structure():
    for name in ("long-pool-b1", "long-pool-b16"):
        w = WORKLOADS[name]
        sb = w.slot_blocks
        assert sb.shape == (w.batch, 1152)
        for b in range(w.batch):
            blocks = sb[b][sb[b] >= 0]
            assert len(np.unique(blocks)) == blocks.size <= 1152
            assert blocks.min() >= 0 and blocks.max() < 4096
            assert blocks.size > 1000            # ~28% of 4096 blocks drawn, pool mostly full
        assert np.array_equal(np.sort(w.block_table.reshape(-1)), np.arange(w.batch * 1152))
        assert np.array_equal(w.block_valid, (sb >= 0).astype(np.uint8))
    # sequence 0 is the same in the batch-1 and batch-16 variants
    assert np.array_equal(WORKLOADS["long-pool-b1"].slot_blocks[0],
                          WORKLOADS["long-pool-b16"].slot_blocks[0])


def test_prefill_workloads_continue_the_ring_workloads():
    """The prefill workloads are the ring workloads' caches, taken a chunk of
    decode steps per call."""
    for pre, ring in (("mha-prefill", "mha-ring"), ("gqa-prefill", "gqa-ring")):
        p, r = WORKLOADS[pre], WORKLOADS[ring]
        assert p.chunk > 0 and p.decode_steps % p.chunk == 0
        assert np.array_equal(p.decode_start, r.decode_start)
        assert p.history_calls()[-1][1] == r.history_calls()[-1][1]
        a = p.rows(TENSOR_K, 1, [7, int(p.decode_start[1]) + 3])
        b = r.rows(TENSOR_K, 1, [7, int(r.decode_start[1]) + 3])
        assert np.array_equal(a, b)

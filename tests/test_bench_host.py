"""Host-side arithmetic of bench.py: the useful-work counts it divides by."""

import numpy as np

import bench
from oracle.ring import resident_positions
from synth import WORKLOADS, RingWorkload


def _ring(W, S):
    return RingWorkload(name="t", seed=0, batch=2, num_q_heads=4, num_kv_heads=2, head_dim=8,
                        dtype="bf16", window=W, sinks=S, rope_base=10000.0, scale=1.0,
                        decode_steps=8, history="prefill:0", chunk=5)


def test_visible_keys_counts_the_resident_set():
    for W, S in ((16, 4), (1, 4), (2, 8), (64, 0), (5, 5)):
        w = _ring(W, S)
        for t in list(range(0, 3 * (W + S))) + [10_000, 2_147_000_000]:
            assert int(bench.visible_keys(w, t)) == len(resident_positions(t, S, W)), (W, S, t)


def test_prefill_flops_sum_rows():
    w = _ring(6, 2)
    first = np.array([0, 40])
    want = sum(len(resident_positions(int(f) + j, 2, 6)) for f in first for j in range(5))
    assert bench.prefill_flops(w, first) == want * 4 * 8 * 4


def test_decode_bytes_of_full_ring():
    w = WORKLOADS["mha-ring"]
    assert bench.resident_tokens(w) == w.batch * w.slots
    assert bench.kv_bytes_per_step(w) == w.batch * w.slots * 2 * 32 * 128 * 2

"""Pins for oracle/kvbytes.py against the values the pages print."""

import os

from oracle.kvbytes import kv_bytes, kv_bytes_per_token, sink_window_bytes
from synth import WORKLOADS

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kv_bytes.txt")


def test_printed_values():
    n = 0
    with open(GOLDEN) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            layers, heads, dim, eb, tokens, batch, want = map(int, line.split())
            assert kv_bytes(tokens, batch, layers, heads, dim, eb) == want
            n += 1
    assert n == 5
    assert kv_bytes_per_token(32, 32, 128, 2) == 524288


def test_gqa_and_mqa_shrink_by_the_head_ratio():
    """[share] §2.2: 32 -> 8 kv heads is 1/4, 32 -> 1 is 1/32."""
    mha = kv_bytes_per_token(32, 32, 128, 2)
    assert kv_bytes_per_token(32, 8, 128, 2) * 4 == mha
    assert kv_bytes_per_token(32, 1, 128, 2) * 32 == mha


def test_sink_window_cache_is_constant_in_stream_length():
    """[sink]: (S + W) slots whatever the stream length."""
    per = kv_bytes_per_token(1, 32, 128, 2)
    assert sink_window_bytes(4, 4096, 1, 32, 128, 2) == 4100 * per


def test_workload_bytes_per_token():
    assert WORKLOADS["mha-ring"].kv_bytes_per_token() == kv_bytes_per_token(1, 32, 128, 2)
    assert WORKLOADS["gqa-ring"].kv_bytes_per_token() == kv_bytes_per_token(1, 8, 128, 2)
    assert WORKLOADS["tiny-ring"].kv_bytes_per_token() == kv_bytes_per_token(1, 4, 64, 4)

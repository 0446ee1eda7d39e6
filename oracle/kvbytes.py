"""KV-cache byte formulas of the pages.

* Per token: 2 (K and V) * layers * kv_heads * head_dim * element bytes
  ([share] §2.2 memory ledger; [kvc] §3.2; [pool] cost formula).
* Sink + window cache: (S + W) * 2 * layers * kv_heads * head_dim * bytes,
  constant in the stream length ([sink], the M_stream formula).
* A ring keeps W entries however long the stream; an append-only list keeps
  all of them ([ring] §4.4: 10,000 tokens with W = 1024).

Pinned by the printed values: 524,288 bytes per token for 32 layers x 32
heads x 128 dims in fp16 ([share] §2.2, [kvc] §3.2), 4 GB at 8192 tokens,
2 GB at 4096 tokens (tests/test_oracle_kvbytes.py).
"""

from __future__ import annotations


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    return 2 * layers * kv_heads * head_dim * elem_bytes


def kv_bytes(tokens: int, batch: int, layers: int, kv_heads: int, head_dim: int,
             elem_bytes: int) -> int:
    return batch * tokens * kv_bytes_per_token(layers, kv_heads, head_dim, elem_bytes)


def sink_window_bytes(sinks: int, window: int, layers: int, kv_heads: int, head_dim: int,
                      elem_bytes: int) -> int:
    return (sinks + window) * kv_bytes_per_token(layers, kv_heads, head_dim, elem_bytes)

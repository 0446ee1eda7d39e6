"""Seeded synthetic inputs for the bounded-KV-cache decode workloads.

This package is shared by the CPU oracle and by the GPU harness (tests,
bench).  It holds none of the method's arithmetic: no RoPE, no slot rule,
no block addressing, no attention.  It only draws raw Q/K/V rows, sequence
lengths, start positions, block tables and residency masks, all from
counter-based seeds so that any position of any sequence can be
re-materialised on its own.
"""

from .draws import (  # noqa: F401
    CHUNK,
    TENSOR_Q,
    TENSOR_K,
    TENSOR_V,
    bf16_bits_from_f32,
    draw_rows,
    draw_rows_parallel,
    encode_storage,
    f32_from_bf16_bits,
)
from .workloads import (  # noqa: F401
    WORKLOADS,
    PagedAppendWorkload,
    PagedWorkload,
    PagerWorkload,
    PoolWorkload,
    RingWorkload,
    workload,
)

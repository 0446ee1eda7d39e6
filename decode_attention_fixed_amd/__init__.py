"""Decode attention over a bounded KV cache (sink + sliding-window ring, paged
pool with validity mask) for MI355X / gfx950.

The compute lives in libswa.so (include/swa.h: C-ABI over hand-written HIP
kernels); `binding` is its thin ctypes layer.  Importing `binding` requires the
built library: build it with `python -m decode_attention_fixed_amd.build`.
"""

__all__ = ["binding", "build"]

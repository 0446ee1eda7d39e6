"""Rotary position embedding at an absolute position, in float64.

The pages ask that the rotation be applied to K before it is cached, at the
token's true (absolute) position, never at its slot index, and that V is not
rotated ([pool] "self-contained shards: bake RoPE into the K rows"; [kvc]
§4.5; [ring] §3.2, §3.4, §6).  They name RoPE without writing it out; the
standard form is used: pairs of coordinates rotated by angle pos * theta_i,
theta_i = base ** (-2 i / d), i < d/2.

Two pairings are offered: "interleaved" pairs (2i, 2i+1), "half" pairs
(i, i + d/2).  The pages fix neither the pairing nor the frequencies, so the
reading is the standard rotary embedding as library implementations define
it, and both are pinned against two of them: GPT-J's interleaved form and
LLaMA's half-split form in `transformers`, frequencies included
(tests/test_oracle_rope_library.py).  Also pinned: rotation at position 0 is
the identity, norms are preserved, d = 2 rotates by `pos` radians, scores
depend only on the position difference, and the two pairings are the same
map up to a fixed coordinate permutation (tests/test_oracle_rope.py).
"""

from __future__ import annotations

import numpy as np


def inv_freq(dim: int, base: float) -> np.ndarray:
    """theta_i = base ** (-2 i / dim), i = 0 .. dim/2 - 1, float64."""
    if dim % 2:
        raise ValueError("head_dim must be even")
    return np.array([float(base) ** (-2.0 * i / dim) for i in range(dim // 2)],
                    dtype=np.float64)


def rope(x, pos, base: float, style: str = "interleaved") -> np.ndarray:
    """Rotate rows x [..., d] at positions pos (broadcast against x[..., 0])."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    theta = inv_freq(d, base)
    angle = np.asarray(pos, dtype=np.float64)[..., None] * theta
    c, s = np.cos(angle), np.sin(angle)
    out = np.empty(np.broadcast_shapes(x.shape, angle.shape[:-1] + (d,)), dtype=np.float64)
    if style == "interleaved":
        a, b = x[..., 0::2], x[..., 1::2]
        out[..., 0::2] = a * c - b * s
        out[..., 1::2] = a * s + b * c
    elif style == "half":
        a, b = x[..., : d // 2], x[..., d // 2:]
        out[..., : d // 2] = a * c - b * s
        out[..., d // 2:] = a * s + b * c
    else:
        raise ValueError(f"unknown rope style {style!r}")
    return out

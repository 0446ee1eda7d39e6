"""int8 KV rows with one scale per row.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing on the product
path imports this module.

[kvc] §5.1 lists quantising the cache from 16 bits to INT8 (half the memory,
a controlled loss of precision, calibration needed) among the ways to shrink
it; the page gives no scheme.  Reading: symmetric absmax quantisation of
every stored row (one head of one token, d values) on its own, so a row is
quantised once when it is written and never again:

    a     = max_i |x_i|                       (x: the row as the cache would
                                               store it, in float64: K rotated
                                               at its position, V as given)
    s     = float32(a / 127)                  (stored next to the codes)
    c_i   = clamp(rint(x_i / s), -127, 127)   (ties to even; s = 0 gives 0)
    x'_i  = c_i * s                           (what attention reads)

The decisions (the float32 scale, the rounding of x_i / s) are taken in
float64 with the float32 scale on both sides, so the codes are reproducible
bit for bit from the same x.  Attention over an int8 cache is attention over
the rows x' (the oracle in oracle/attention.py, float64).

Pins (tests/test_oracle_quant.py): rows that are exact multiples of a
power-of-two scale with a largest code of 127 come back exactly; every
element is within s / 2 of its row (s / 2 + the clamp for none, since
|x_i| <= a); the largest |code| is 127 at the largest |x_i|; quant(-x) =
-quant(x); a zero row gives scale 0 and codes 0; the code is the nearest
integer to x_i / s by brute force over all 255 codes (ties to even).
"""

from __future__ import annotations

import numpy as np


def quantize_rows(x) -> tuple:
    """(codes int8 [..., d], scales float32 [...]) of rows x [..., d] (float64)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x).max(axis=-1)
    s = (a / 127.0).astype(np.float32)
    s64 = s.astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s64 > 0, np.rint(x / np.where(s64 > 0, s64, 1.0)), 0.0)
    return np.clip(q, -127, 127).astype(np.int8), s


def dequantize_rows(codes, scales) -> np.ndarray:
    """Rows x' = code * scale, float64."""
    return np.asarray(codes, dtype=np.float64) * np.asarray(scales, dtype=np.float64)[..., None]


def quantize_dequantize(x) -> np.ndarray:
    return dequantize_rows(*quantize_rows(x))

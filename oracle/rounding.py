"""Rounding of float64 results to the cache's storage dtypes.

Storing a rotated K row (or query) in bf16 or float32 is a rounding to
nearest, ties to even, of the exact rotated value (the pages do not state a
rounding; this is IEEE's default).  Written from the definition: scale by the
power of two that puts the target format's last mantissa bit at 1, round
half-even to an integer, scale back.

Pins (tests/test_oracle_rounding.py): exact rational rounding with Python
fractions on random and tie-constructed values, torch's float32 -> bf16
conversion for inputs that are float32 values, numpy's float32 cast.
"""

from __future__ import annotations

import numpy as np

_BF16_MANT = 8          # significant bits, including the implicit one
_BF16_MIN_EXP = -125    # frexp exponent of the smallest normal bf16 (2**-126)
_BF16_MAX = float.fromhex("0x1.fep127")


def round_bf16(x) -> np.ndarray:
    """float64 -> nearest bf16 value (ties to even), returned as float64."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    e = np.maximum(e, _BF16_MIN_EXP)
    quantum = np.ldexp(1.0, e - _BF16_MANT)
    y = np.rint(x / quantum) * quantum
    if np.any(np.abs(y[np.isfinite(x)]) > _BF16_MAX):
        raise OverflowError("value outside the bf16 range")
    return y


def round_f32(x) -> np.ndarray:
    """float64 -> nearest float32 value (ties to even), returned as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_store(x, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f32":
        return round_f32(x)
    raise ValueError(dtype)


def bf16_bits(x) -> np.ndarray:
    """Bit patterns of values that are exactly representable in bf16."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)

"""Storage-type conversions used by the oracle (test infrastructure).

bfloat16 is kept as uint16 bit patterns: the upper half of an IEEE binary32.
Upcasting is exact.  Downcasting rounds to nearest, ties to even, which is the
rounding the rotary embedding's output uses ([WF] §4.2 publishes RoPE'd K in
the model's storage type; the pages do not name the rounding, and round to
nearest even is the reading taken).
"""
from __future__ import annotations

import numpy as np


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact upcast of bfloat16 bit patterns to float32."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bits, round to nearest with ties to even.

    Adding 0x7FFF plus the lowest kept bit to the 32-bit pattern and keeping
    the upper half rounds the discarded 16 bits to nearest; on an exact tie
    the kept bit decides, which yields the even neighbour.  NaN stays NaN
    (quiet bit forced so the truncation cannot produce an infinity).
    """
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32)
    keep_lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = ((u + np.uint32(0x7FFF) + keep_lsb) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        rounded = np.where(nan, ((u >> np.uint32(16)) | np.uint32(0x0040)).astype(np.uint16),
                           rounded)
    return rounded


def to_f32(values: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array (uint16 bits for bf16, float32 for fp32) -> float32."""
    if dtype == "bf16":
        return bf16_to_f32(values)
    return np.asarray(values, dtype=np.float32)


def from_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 -> storage array of `dtype`."""
    if dtype == "bf16":
        return f32_to_bf16(x)
    return np.asarray(x, dtype=np.float32)

"""Storage-dtype conversions of the oracle (test infrastructure only).

Inputs reach the oracle as NumPy arrays: fp16 as ``np.float16``, bf16 as the raw
``np.uint16`` bit patterns (NumPy has no bf16 type), fp32 as ``np.float32``.

* fp16/bf16 -> fp32 is exact.
* fp32 -> bf16 rounds to nearest, ties to even, written out on the bit pattern:
  keep the high 16 bits after adding 0x7FFF plus the lowest kept bit.
* fp32 -> fp16 rounds to nearest even (IEEE conversion).
"""
from __future__ import annotations

import numpy as np

F16, BF16, F32 = "fp16", "bf16", "fp32"


def bf16_bits_to_f32(u16: np.ndarray) -> np.ndarray:
    u = np.asarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32)


def f32_to_bf16_bits(f: np.ndarray) -> np.ndarray:
    f = np.asarray(f, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    return np.where(np.isnan(f), np.uint16(0x7FC0), r).astype(np.uint16)


def to_f32(a: np.ndarray, dtype: str) -> np.ndarray:
    """Decode a storage array to float32 (exact)."""
    if dtype == BF16:
        return bf16_bits_to_f32(a)
    if dtype == F16:
        return np.asarray(a, dtype=np.float16).astype(np.float32)
    if dtype == F32:
        return np.asarray(a, dtype=np.float32)
    raise ValueError(dtype)


def from_f32(f: np.ndarray, dtype: str) -> np.ndarray:
    """Encode float32 values in a storage dtype (RNE)."""
    f = np.asarray(f, dtype=np.float32)
    if dtype == BF16:
        return f32_to_bf16_bits(f)
    if dtype == F16:
        return f.astype(np.float16)
    if dtype == F32:
        return f.copy()
    raise ValueError(dtype)

"""Storage formats and rounding used by the oracle (fp16 / bf16 patterns, directed fp16 rounding).

bf16 is the upper half of an IEEE-754 binary32; fp16 is IEEE-754 binary16. All conversions here are written
from those definitions (bf16 round-to-nearest-even by integer arithmetic on the binary32 pattern; fp16 through
numpy's binary16, which rounds to nearest even).
"""
from __future__ import annotations

import numpy as np


def storage_to_f32(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of 16-bit storage patterns to float32."""
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float32)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    raise ValueError(dtype)


def storage_to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    return storage_to_f32(bits, dtype).astype(np.float64)


def f32_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 pattern, round to nearest, ties to even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def f32_to_storage_rne(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f32_to_bf16_rne(x)
    if dtype == "f16":
        return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)
    raise ValueError(dtype)


def f16_round_down(x: np.ndarray) -> np.ndarray:
    """Largest binary16 value <= x (x float32, |x| < 65504). Returns float16."""
    x = np.asarray(x, dtype=np.float32)
    f = x.astype(np.float16)
    above = f.astype(np.float32) > x
    return np.where(above, np.nextafter(f, np.float16(-np.inf)), f).astype(np.float16)


def f16_round_up(x: np.ndarray) -> np.ndarray:
    """Smallest binary16 value >= x (x float32, |x| < 65504). Returns float16."""
    x = np.asarray(x, dtype=np.float32)
    f = x.astype(np.float16)
    below = f.astype(np.float32) < x
    return np.where(below, np.nextafter(f, np.float16(np.inf)), f).astype(np.float16)

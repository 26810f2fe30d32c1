"""INT2 recoverable tier: group quantiser, dequantiser and code packing.

Source: QEvict page, "Metodologia: QEvict" (recoverable quantized tier, INT2 in the experiments) and
"Mecanismos Principais" (write-once quantization ledger). The page gives the bit width only; the group format is
a reading, written out here:

  * a group is 32 contiguous head_dim elements of one token (4 groups per 128-dim row), for K and V alike;
  * lo, hi = min / max of the group, exact in fp32;
  * zero  z = the largest fp16 value <= lo;
  * scale s = the smallest fp16 value >= fl32(fl32(hi - z) / 3), or 0 when hi == z;
  * code  c = #{k in {0, 1, 2} : fl32(x - z) >= (k + 1/2) * s}, and c = 0 when s == 0
    (nearest of the four levels z, z+s, z+2s, z+3s, ties upward; the products (k+1/2)*s are exact in fp32);
  * dequantised value x^ = fl32(c*s + z) (c*s + z is exact before the one rounding, i.e. an fp32 fma).

These decisions are integers, so they are taken in fp32 just as the GPU takes them.

Packing: four codes per byte, element 4b + j of a row in bits 2j..2j+1 of byte b; the group metadata is one
32-bit word per (token, group) holding the fp16 scale in bits 0..15 and the fp16 zero in bits 16..31.
"""
from __future__ import annotations

import numpy as np

from .fp import f16_round_down, f16_round_up, storage_to_f32

GROUP = 32


def quantize(bits: np.ndarray, dtype: str):
    """Quantise rows of storage-dtype values. bits [..., D] -> (codes uint8 [..., D], s f16 [..., D/32],
    z f16 [..., D/32])."""
    x = storage_to_f32(bits, dtype)
    D = x.shape[-1]
    g = x.reshape(x.shape[:-1] + (D // GROUP, GROUP))
    lo = g.min(axis=-1)
    hi = g.max(axis=-1)
    z16 = f16_round_down(lo)
    z = z16.astype(np.float32)
    span = (hi - z).astype(np.float32)
    t = (span / np.float32(3.0)).astype(np.float32)
    flat = hi == z
    s16 = np.where(flat, np.float16(0.0), f16_round_up(np.where(flat, np.float32(1.0), t))).astype(np.float16)
    s = s16.astype(np.float32)
    diff = (g - z[..., None]).astype(np.float32)
    codes = np.zeros(g.shape, np.uint8)
    for k in range(3):
        thr = (np.float32(k + 0.5) * s).astype(np.float32)
        codes += (diff >= thr[..., None]).astype(np.uint8)
    codes = np.where((s == 0)[..., None], np.uint8(0), codes).astype(np.uint8)
    return codes.reshape(x.shape), s16, z16


def dequantize(codes: np.ndarray, s16: np.ndarray, z16: np.ndarray) -> np.ndarray:
    """x^ = fl32(c*s + z) (exact c*s + z in fp64, then one rounding to fp32). Returns float32 [..., D]."""
    D = codes.shape[-1]
    c = codes.reshape(codes.shape[:-1] + (D // GROUP, GROUP)).astype(np.float64)
    exact = c * s16.astype(np.float64)[..., None] + z16.astype(np.float64)[..., None]
    return exact.astype(np.float32).reshape(codes.shape)


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """[..., D] codes (0..3) -> [..., D/4] bytes; element 4b+j in bits 2j..2j+1 of byte b."""
    c = codes.reshape(codes.shape[:-1] + (codes.shape[-1] // 4, 4)).astype(np.uint8)
    out = np.zeros(c.shape[:-1], np.uint8)
    for j in range(4):
        out |= (c[..., j] & 3) << (2 * j)
    return out


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.stack([(p >> (2 * j)) & 3 for j in range(4)], axis=-1)
    return out.reshape(p.shape[:-1] + (p.shape[-1] * 4,)).astype(np.uint8)


def pack_meta(s16: np.ndarray, z16: np.ndarray) -> np.ndarray:
    """(scale, zero) fp16 pairs -> uint32 words: scale in bits 0..15, zero in bits 16..31."""
    s = np.asarray(s16, dtype=np.float16).view(np.uint16).astype(np.uint32)
    z = np.asarray(z16, dtype=np.float16).view(np.uint16).astype(np.uint32)
    return (s | (z << np.uint32(16))).astype(np.uint32)


def unpack_meta(meta: np.ndarray):
    m = np.asarray(meta, dtype=np.uint32)
    s = (m & np.uint32(0xFFFF)).astype(np.uint16).view(np.float16)
    z = (m >> np.uint32(16)).astype(np.uint16).view(np.float16)
    return s, z

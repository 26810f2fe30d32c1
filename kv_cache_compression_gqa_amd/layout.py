"""Host-side conversions between logical arrays and the library's storage layouts (include/kvc.h).

Logical arrays are indexed [..., token, head_dim] (codes as one uint8 0..3 per element, scale/zero as fp16).
Library layouts:
  V window       [D][W]            (head_dim-major inside a window)
  V tail         [TM/32][D][32]    (head_dim-major inside each 32-token block)
  K codes row    32 bytes per token; byte 8*s + 2*g + h holds head_dim 32g + 8s + 4h + e at bits 2e
  K meta         [W][4] words      (fp16 scale in bits 0..15, fp16 zero in bits 16..31)
  V codes        [16][4][8] 16-bit words per window; word (r, q, dt) holds tokens 8q + e of head_dim 16dt + r at
                 bits 2e
  V meta         [4][4][8] words per window; word (q, g, e) = token 8q + e, group g
Only index permutations live here; no arithmetic of the method.
"""
from __future__ import annotations

import numpy as np

W, D = 32, 128


def v_win_to_lib(v: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(np.swapaxes(v, -1, -2))


def v_win_from_lib(v: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(np.swapaxes(v, -1, -2))


def v_tail_to_lib(v: np.ndarray) -> np.ndarray:
    """[..., TM, D] -> [..., TM/32, D, 32]"""
    TM = v.shape[-2]
    assert TM % W == 0
    x = v.reshape(v.shape[:-2] + (TM // W, W, D))
    return np.ascontiguousarray(np.swapaxes(x, -1, -2))


def v_tail_from_lib(v: np.ndarray) -> np.ndarray:
    x = np.swapaxes(v, -1, -2)
    return np.ascontiguousarray(x.reshape(x.shape[:-3] + (x.shape[-3] * W, D)))


def k_codes_to_lib(codes: np.ndarray) -> np.ndarray:
    """[..., W, D] codes -> [..., W, 32] bytes."""
    c = np.asarray(codes, np.uint8)
    out = np.zeros(c.shape[:-1] + (32,), np.uint8)
    for g in range(4):
        for s in range(4):
            for h in range(2):
                byte = np.zeros(c.shape[:-1], np.uint8)
                for e in range(4):
                    byte |= (c[..., 32 * g + 8 * s + 4 * h + e] & 3) << (2 * e)
                out[..., 8 * s + 2 * g + h] = byte
    return out


def k_codes_from_lib(b: np.ndarray) -> np.ndarray:
    b = np.asarray(b, np.uint8)
    out = np.zeros(b.shape[:-1] + (D,), np.uint8)
    for g in range(4):
        for s in range(4):
            for h in range(2):
                for e in range(4):
                    out[..., 32 * g + 8 * s + 4 * h + e] = (b[..., 8 * s + 2 * g + h] >> (2 * e)) & 3
    return out


def v_codes_to_lib(codes: np.ndarray) -> np.ndarray:
    """[..., W, D] codes -> [..., 16, 4, 8] uint16 words."""
    c = np.asarray(codes, np.uint16)
    out = np.zeros(c.shape[:-2] + (16, 4, 8), np.uint16)
    for r in range(16):
        for q in range(4):
            for dt in range(8):
                word = np.zeros(c.shape[:-2], np.uint16)
                for e in range(8):
                    word |= (c[..., 8 * q + e, 16 * dt + r] & 3) << (2 * e)
                out[..., r, q, dt] = word
    return out


def v_codes_from_lib(words: np.ndarray) -> np.ndarray:
    w = np.asarray(words, np.uint16)
    out = np.zeros(w.shape[:-3] + (W, D), np.uint8)
    for r in range(16):
        for q in range(4):
            for dt in range(8):
                for e in range(8):
                    out[..., 8 * q + e, 16 * dt + r] = (w[..., r, q, dt] >> (2 * e)) & 3
    return out


def meta_words(s16: np.ndarray, z16: np.ndarray) -> np.ndarray:
    s = np.asarray(s16, np.float16).view(np.uint16).astype(np.uint32)
    z = np.asarray(z16, np.float16).view(np.uint16).astype(np.uint32)
    return (s | (z << np.uint32(16))).astype(np.uint32)


def k_meta_to_lib(s16: np.ndarray, z16: np.ndarray) -> np.ndarray:
    """[..., W, 4] fp16 pairs -> [..., W, 4] words."""
    return meta_words(s16, z16)


def v_meta_to_lib(s16: np.ndarray, z16: np.ndarray) -> np.ndarray:
    """[..., W, 4] fp16 pairs -> [..., 4 (q), 4 (g), 8 (e)] words."""
    m = meta_words(s16, z16)                                  # [..., 32, 4]
    m = m.reshape(m.shape[:-2] + (4, 8, 4))                   # [..., q, e, g]
    return np.ascontiguousarray(np.swapaxes(m, -1, -2))       # [..., q, g, e]

"""Decode attention over a per-head variable-length paged cache, written out in fp64 (test infrastructure: only the
tests, the smoke check and the benchmark's CPU baseline use this module).

Source: DBTrimKV page ("Make Each Token Count: Towards Improving Long-Context Performance with KV Cache
Eviction"), "Metodologia: Evicção Baseada em Retenção Global", section 4: after the global budget, every head
keeps a sequence of its own length in a PagedAttention layout, and decoding attends over that head's kept
tokens only. A row (one (layer, KV head) pair) lists its pages in order; token i of the row is row i % page of
pool page page_list[i // page]. The G query heads of the row attend with standard scaled dot-product attention
(the same definition as the decode attention of the QEvict page).

Readings:
  * token order inside the row is list order, so position i of the kept sequence is the i-th listed row;
  * rows past the length on the last page are not keys (they are never read);
  * a row of length 0 has no keys: its output is defined as zeros.
"""
from __future__ import annotations

import numpy as np

from .attention import gqa_decode


def gather_row(pool: np.ndarray, page_list: np.ndarray, length: int, page: int) -> np.ndarray:
    """pool [n_pages][page][D], page_list [>= ceil(length/page)] -> the row's keys (or values) [length][D]."""
    rows = []
    for i in range(length):
        rows.append(pool[int(page_list[i // page]), i % page])
    D = pool.shape[-1]
    return np.array(rows, dtype=pool.dtype).reshape(length, D)


def paged_gqa_decode(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray, page_list: np.ndarray, length: int,
                     page: int) -> np.ndarray:
    """q [G][D] and the pools (fp64 values) -> o [G][D] over the row's ``length`` tokens (zeros if length == 0)."""
    G, D = q.shape
    if length == 0:
        return np.zeros((G, D), np.float64)
    K = gather_row(k_pool, page_list, length, page).astype(np.float64)
    V = gather_row(v_pool, page_list, length, page).astype(np.float64)
    return gqa_decode(q, K, V)[2]

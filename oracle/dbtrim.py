"""DBTrimKV global retention budget and per-head paged compaction.

Source: DBTrimKV page ("Make Each Token Count: Towards Improving Long-Context Performance with KV Cache
Eviction"), "Metodologia: Evicção Baseada em Retenção Global" —
  * section 2: the retention weight of token i at step t is r_{t,i} = beta_i^(t - i);
  * section 3: one global budget M_global; at an eviction step every cached entry of every layer and head is
    ranked by predicted future utility on one common scale and the top M_global are kept;
  * section 4: PagedAttention layout so that each head keeps a variable-length sequence.

Readings:
  * ranking uses log r = (t - i) * ln(beta_i) (a monotone map of r, so the order is the same); literal
    beta^(t-i) underflows to 0 for most entries at t = 131072 and would leave the order to tie-breaks;
  * i is 0-based, t = n_tokens, so t - i runs over [1, n_tokens];
  * global order (score desc, flat index asc), flat = (layer * H + head) * n_tokens + i;
  * compaction is out of place: per (layer, head) the kept positions in ascending order are packed into fresh
    pages of ``page`` rows, page ids consecutive in (layer, head) order, the last page of a head partially
    filled and its unused rows zero.
"""
from __future__ import annotations

import numpy as np

from .select import global_topm


def log_retention(beta: np.ndarray, t: int) -> np.ndarray:
    """beta [L][H][T] float32 -> (t - i) * ln(beta) in fp64, same shape."""
    T = beta.shape[-1]
    age = (t - np.arange(T)).astype(np.float64)
    return age * np.log(beta.astype(np.float64))


def keep_mask(scores: np.ndarray, m: int) -> np.ndarray:
    return global_topm(scores.reshape(-1), m).reshape(scores.shape)


def compact_plan(keep: np.ndarray, page: int):
    """keep [L][H][T] bool -> (lengths [L*H], page_offset [L*H], n_pages [L*H], positions list per head)."""
    L, H, T = keep.shape
    lengths = keep.reshape(L * H, T).sum(axis=1).astype(np.int64)
    n_pages = (lengths + page - 1) // page
    page_offset = np.concatenate([[0], np.cumsum(n_pages)[:-1]]).astype(np.int64)
    positions = [np.flatnonzero(keep.reshape(L * H, T)[lh]) for lh in range(L * H)]
    return lengths, page_offset, n_pages, positions


def compact_rows(keep: np.ndarray, page_table: np.ndarray, page: int):
    """Source pool row for every destination row: returns (dst_rows_total, src_row [n_dst_pages*page] with -1
    for the zero rows of partial pages), plus the plan."""
    L, H, T = keep.shape
    lengths, page_offset, n_pages, positions = compact_plan(keep, page)
    total_pages = int(n_pages.sum())
    src = np.full(total_pages * page, -1, np.int64)
    pt = page_table.reshape(L * H, -1).astype(np.int64)
    for lh in range(L * H):
        pos = positions[lh]
        rows = pt[lh][pos // page] * page + pos % page
        start = int(page_offset[lh]) * page
        src[start:start + pos.size] = rows
    return src, lengths, page_offset, n_pages

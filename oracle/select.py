"""Budgeted selection: ranking, three-tier routing, two-stage selection, global top-M.

Every ranking is by (score descending, index ascending): ties go to the lower index, which makes every selection
unique. NaN scores are rejected.

Sources:
  * three tiers under a fixed budget — QEvict page, "Metodologia: QEvict" (full precision / recoverable
    quantized / evicted) and "Mecanismos Principais" (demotion, promotion);
  * two-stage selection — CriticalKV page, "Algoritmo: Seleção Constrainda por Perturbação" (Algorithm 1):
    b' = alpha*b entries by attention weight, the remaining b'' = b - b' by A_i * |V_i W_O|_1;
  * global top-M — DBTrimKV page ("Make Each Token Count"), "Metodologia" section 3: rank every cached entry
    of every layer and head on one scale and keep the top M_global.
"""
from __future__ import annotations

import math

import numpy as np

FULL, INT2, EVICTED = 0, 1, 2


def rank_order(scores: np.ndarray) -> np.ndarray:
    """Indices of ``scores`` ordered by (score desc, index asc)."""
    sc = np.asarray(scores, dtype=np.float64)
    if np.isnan(sc).any():
        raise ValueError("NaN score")
    idx = np.arange(sc.size)
    return np.lexsort((idx, -sc))


def topk(scores: np.ndarray, k: int) -> np.ndarray:
    """First k indices of the (score desc, index asc) order."""
    return rank_order(scores)[:k]


def three_tier(scores: np.ndarray, tier: np.ndarray, b_full: int, b_int2: int) -> np.ndarray:
    """New tier per window. Resident windows (tier != EVICTED) are ranked; ranks [0, b_full) become FULL,
    [b_full, b_full + b_int2) INT2, the rest EVICTED. Evicted windows stay evicted."""
    tier = np.asarray(tier)
    res = np.flatnonzero(tier != EVICTED)
    order = res[rank_order(np.asarray(scores, dtype=np.float64)[res])]
    new = np.full(tier.shape, EVICTED, dtype=np.int8)
    new[order[:b_full]] = FULL
    new[order[b_full:b_full + b_int2]] = INT2
    return new


def two_stage(a: np.ndarray, s2: np.ndarray, budget: int, alpha: float) -> np.ndarray:
    """Stage 1: top floor(alpha*b) by a. Stage 2: top (b - b') by s2 among the rest. Sorted ascending."""
    b1 = int(math.floor(alpha * budget))
    i1 = topk(a, b1)
    taken = np.zeros(np.asarray(a).size, bool)
    taken[i1] = True
    order2 = rank_order(s2)
    i2 = order2[~taken[order2]][:budget - b1]
    return np.sort(np.concatenate([i1, i2]))


def global_topm(scores_flat: np.ndarray, m: int) -> np.ndarray:
    """Boolean keep mask of the first m entries in (score desc, flat index asc) order."""
    keep = np.zeros(np.asarray(scores_flat).size, bool)
    keep[topk(scores_flat, m)] = True
    return keep

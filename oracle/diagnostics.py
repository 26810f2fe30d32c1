"""Routing diagnostics of a compressed-cache decode run, written out in fp64 (test infrastructure: only the tests,
the smoke check and the benchmark's CPU baseline use this module).

Sources:
  * QEvict page ("Resumo Técnico: QEvict"), "Principais Contribuições", item 1: three diagnostics of cache
    dynamics under a policy: the future missed mass (the share of later attention that falls on states the policy
    has already dropped), global latent importance reactivation (how often windows that had gone inactive come
    back into the active set) and selection churn (how unstable the assignments are from one routing step to the
    next);
  * CriticalKV page ("Resumo Técnico: CriticalKV"), "Framework Teórico": the output perturbation L is the L1
    distance between the attention output over the full cache and over the kept subset.

Readings (the pages give the quantities in prose only):
  * future missed mass at a decode step = the full-cache attention mass (mean over the G query heads of the
    probability, as for the window score) on the windows that are EVICTED in the tiers serving that step;
  * the active set is the FULL tier. Every window starts FULL, so a window that enters the FULL tier at an event
    has been active before: re-entries at an event = windows FULL after it and not FULL before it (promotions);
    global LIR over a run = re-entries summed over events / FULL windows summed over events;
  * churn at an event = the windows whose tier changed, over the unit's windows;
  * L = sum over head_dim of |o - o^| per query head, o over the full cache and o^ over the compressed one.
"""
from __future__ import annotations

import numpy as np

from .select import EVICTED, FULL


def route_counts(tier_prev: np.ndarray, tier: np.ndarray) -> tuple[int, int, int, int]:
    """(changed, re-entered FULL, FULL, resident) over the windows of one unit."""
    a = np.asarray(tier_prev)
    b = np.asarray(tier)
    changed = int(np.count_nonzero(a != b))
    reentered = int(np.count_nonzero((b == FULL) & (a != FULL)))
    return changed, reentered, int(np.count_nonzero(b == FULL)), int(np.count_nonzero(b != EVICTED))


def future_missed_mass(mass_full: np.ndarray, tier: np.ndarray) -> float:
    """Full-cache window mass on the windows evicted in ``tier``."""
    m = np.asarray(mass_full, np.float64)
    return float(m[np.asarray(tier) == EVICTED].sum())


def perturbation_l1(o_full: np.ndarray, o: np.ndarray) -> np.ndarray:
    """[G]: sum_d |o_full[h, d] - o[h, d]|."""
    return np.abs(np.asarray(o_full, np.float64) - np.asarray(o, np.float64)).sum(axis=1)


def churn(tier_prev: np.ndarray, tier: np.ndarray) -> float:
    return route_counts(tier_prev, tier)[0] / max(1, np.asarray(tier).size)


def global_lir(events) -> float:
    """events: iterable of (tier_prev, tier) pairs of one run -> re-entries / FULL windows, both summed."""
    re = full = 0
    for a, b in events:
        c = route_counts(a, b)
        re += c[1]
        full += c[2]
    return re / full if full else 0.0

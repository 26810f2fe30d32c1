"""Grouped-query decode attention and window mass, written out in fp64.

Source: QEvict page, "Mecanismos Principais": window importance is attention accumulated over time, attention is
materialised to compute it, and grouped-query attention is supported. Standard scaled dot-product attention:
s_{h,i} = q_h . k_i / sqrt(D), p_h = softmax_i(s_h), o_h = sum_i p_{h,i} v_i, for the G query heads h that share
one KV head. Window mass (reading of the GQA aggregation, which the page leaves open): the mean over the G heads
of the probability that falls in the window, mass_w = (1/G) sum_h sum_{i in w} p_{h,i}.

Weighted window score: the CriticalKV page ("Algoritmo") describes its perturbation-constrained score as a plug-in
for existing accumulation pipelines: a key's attention weight is multiplied by the L1 norm of its value projected
through W_O. Inside QEvict's window score that gives mass_w = (1/G) sum_h sum_{i in w} p_{h,i} n_{h,i}, with
n_{h,i} = |V_i W_O,h|_1 for query head h (the group mean of the per-head product, as for CriticalKV's own score).
"""
from __future__ import annotations

import math

import numpy as np


def gqa_decode(q: np.ndarray, K: np.ndarray, V: np.ndarray, bias=None):
    """q [G][D], K [n][D], V [n][D] (fp64) -> (logits [G][n], p [G][n], o [G][D]). ``bias`` [n] (optional) is
    added to every head's logits (the size correction of summary keys)."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    D = q.shape[-1]
    s = (q @ K.T) / math.sqrt(D)
    if bias is not None:
        s = s + np.asarray(bias, dtype=np.float64)[None, :]
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    p = e / e.sum(axis=1, keepdims=True)
    o = p @ V
    return s, p, o


def window_mass(p: np.ndarray, key_window: np.ndarray, n_windows: int) -> np.ndarray:
    """p [G][n], key_window [n] (window id, or -1 for keys outside any window) -> mass [n_windows]."""
    G = p.shape[0]
    per_key = p.sum(axis=0) / G
    mass = np.zeros(n_windows, np.float64)
    sel = key_window >= 0
    np.add.at(mass, key_window[sel], per_key[sel])
    return mass


def weighted_window_mass(p: np.ndarray, key_pos: np.ndarray, weight: np.ndarray, n_windows: int,
                         window: int) -> np.ndarray:
    """p [G][n], key_pos [n] (cache position of each key, -1 for keys outside any window), weight [G][>= n_windows
    * window] (per query head and position) -> mass [n_windows] = (1/G) sum_h sum_{keys in w} p[h] * weight[h]."""
    G = p.shape[0]
    mass = np.zeros(n_windows, np.float64)
    for j in range(p.shape[1]):
        pos = int(key_pos[j])
        if pos < 0:
            continue
        acc = 0.0
        for h in range(G):
            acc += p[h, j] * float(weight[h, pos])
        mass[pos // window] += acc / G
    return mass

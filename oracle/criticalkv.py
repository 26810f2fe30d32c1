"""CriticalKV scores and two-stage selection for one layer at prefill.

Source: CriticalKV page ("Resumo Técnico: CriticalKV") —
  * "Framework Teórico": the output perturbation L = |o - o^|_1 is bounded through the attention weights A and
    the projected values V W_O, W_O being the output projection;
  * "Algoritmo: Seleção Constrainda por Perturbação" (Algorithm 1): stage 1 spends b' = alpha*b (alpha = 0.5)
    on the entries of highest attention weight; stage 2 spends the remaining b'' on the entries that maximise
    A_i * |V_i W_O|_1 (the printed formula drops W_O; the surrounding text and the bound are about the projected
    values, so the projected norm is used); the host method's own accumulation (SnapKV-style observation window)
    is kept.

Readings:
  * observation window = the n_obs trailing prompt positions; query j (position n - n_obs + j) sees keys
    0 .. n - n_obs + j (causal);
  * A_{h,i} = (1/n_obs) * sum_j p_{h,j,i} (masked entries count 0);
  * N_{h,i} = sum_c | sum_d V_{g,i,d} * W_O[h*D + d, c] |, W_O stored [input feature][output feature];
  * per KV head g (budget per KV head): A_g = mean over the G query heads of A_{h,.},
    S2_g = mean over the G heads of A_{h,.} * N_{h,.}.
"""
from __future__ import annotations

import math

import numpy as np

from .select import two_stage


def observation_attention(q_obs: np.ndarray, k: np.ndarray, group: int) -> np.ndarray:
    """q_obs [Hq][T][D], k [Hkv][n][D] (fp64) -> A [Hq][n] fp64."""
    Hq, T, D = q_obs.shape
    n = k.shape[1]
    A = np.zeros((Hq, n), np.float64)
    pos = n - T + np.arange(T)
    allowed = np.arange(n)[None, :] <= pos[:, None]       # [T][n]
    for h in range(Hq):
        s = (q_obs[h] @ k[h // group].T) / math.sqrt(D)    # [T][n]
        s = np.where(allowed, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        e = np.where(allowed, np.exp(s - m), 0.0)
        p = e / e.sum(axis=1, keepdims=True)
        A[h] = p.sum(axis=0) / T
    return A


def projected_value_l1(v_g: np.ndarray, w_o_h: np.ndarray) -> np.ndarray:
    """v_g [n][D], w_o_h [D][d_model] (fp64) -> N [n] = |v_i W_O,h|_1."""
    return np.abs(v_g @ w_o_h).sum(axis=1)


def scores(q_obs: np.ndarray, k: np.ndarray, v: np.ndarray, w_o: np.ndarray, group: int, rows=None):
    """Returns (A [Hq][n], N [Hq][n'] , A_g [Hkv][n], S2_g [Hkv][n'] ) with n' = n, or the listed rows only."""
    Hq, _, D = q_obs.shape
    Hkv, n, _ = k.shape
    A = observation_attention(q_obs, k, group)
    rows = np.arange(n) if rows is None else np.asarray(rows)
    N = np.zeros((Hq, rows.size), np.float64)
    for h in range(Hq):
        N[h] = projected_value_l1(v[h // group][rows], w_o[h * D:(h + 1) * D])
    A_g = A.reshape(Hkv, group, n).mean(axis=1)
    S2_g = (A[:, rows] * N).reshape(Hkv, group, rows.size).mean(axis=1)
    return A, N, A_g, S2_g


def select(A_g: np.ndarray, S2_g: np.ndarray, budget: int, alpha: float) -> np.ndarray:
    """Per KV head two-stage selection -> [Hkv][budget] ascending indices."""
    return np.stack([two_stage(A_g[g], S2_g[g], budget, alpha) for g in range(A_g.shape[0])])

"""Pins for the oracle's CriticalKV scores/selection and DBTrimKV retention/compaction (CPU only)."""
import math

import mpmath
import numpy as np
from hypothesis import given, settings, strategies as st

from oracle import criticalkv, dbtrim, select


def test_observation_attention_causal_mask_by_loops():
    rng = np.random.default_rng(9)
    Hq, G, T, n, D = 4, 2, 3, 7, 4
    q = rng.standard_normal((Hq, T, D))
    k = rng.standard_normal((Hq // G, n, D))
    A = criticalkv.observation_attention(q, k, G)
    for h in range(Hq):
        acc = [0.0] * n
        for j in range(T):
            last = n - T + j                     # query j sits at position n - T + j, sees keys 0..last
            s = [sum(q[h, j, d] * k[h // G, i, d] for d in range(D)) / math.sqrt(D) for i in range(last + 1)]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            tot = math.fsum(e)
            for i in range(last + 1):
                acc[i] += e[i] / tot / T
        np.testing.assert_allclose(A[h], acc, rtol=1e-12, atol=1e-15)
        assert abs(A[h].sum() - 1.0) < 1e-12
    # the last key is seen only by the last query
    assert np.all(A[:, n - 1] <= 1.0 / T + 1e-15)


def test_projected_norm_by_loops_and_identity():
    rng = np.random.default_rng(10)
    v = rng.standard_normal((5, 4))
    w = rng.standard_normal((4, 6))
    N = criticalkv.projected_value_l1(v, w)
    for i in range(5):
        ref = math.fsum(abs(math.fsum(v[i, d] * w[d, c] for d in range(4))) for c in range(6))
        assert abs(N[i] - ref) < 1e-12
    np.testing.assert_allclose(criticalkv.projected_value_l1(v, np.eye(4)), np.abs(v).sum(axis=1), rtol=1e-15)


def test_criticalkv_scores_group_means():
    rng = np.random.default_rng(11)
    Hq, G, T, n, D, dm = 4, 2, 4, 40, 8, 16
    q, k, v = rng.standard_normal((Hq, T, D)), rng.standard_normal((Hq // G, n, D)), rng.standard_normal(
        (Hq // G, n, D))
    w = rng.standard_normal((Hq * D, dm))
    A, N, A_g, S2_g = criticalkv.scores(q, k, v, w, G)
    for g in range(Hq // G):
        np.testing.assert_allclose(A_g[g], (A[2 * g] + A[2 * g + 1]) / 2, rtol=1e-15)
        np.testing.assert_allclose(S2_g[g], (A[2 * g] * N[2 * g] + A[2 * g + 1] * N[2 * g + 1]) / 2, rtol=1e-15)
    # sampled rows give the same values
    rows = np.array([0, 7, 39])
    _, N2, _, S2b = criticalkv.scores(q, k, v, w, G, rows=rows)
    np.testing.assert_allclose(N2, N[:, rows], rtol=1e-15)
    np.testing.assert_allclose(S2b, S2_g[:, rows], rtol=1e-15)
    sel = criticalkv.select(A_g, S2_g, 10, 0.5)
    assert sel.shape == (2, 10) and all(len(set(r)) == 10 and list(r) == sorted(r) for r in sel)


@settings(max_examples=40, deadline=None)
@given(st.integers(0, 2 ** 31 - 1))
def test_log_retention_order_equals_exact_power_order(seed):
    rng = np.random.default_rng(seed)
    T = 24
    beta = np.clip(rng.beta(8, 2, size=(1, 2, T)), 2 ** -24, 1 - 2 ** -24).astype(np.float32)
    s = dbtrim.log_retention(beta, T).reshape(-1)
    mpmath.mp.dps = 60
    exact = [mpmath.power(mpmath.mpf(float(b)), T - (i % T)) for i, b in enumerate(beta.reshape(-1))]
    ref = sorted(range(len(exact)), key=lambda i: (-exact[i], i))
    got = list(select.rank_order(s))
    assert got == ref


def test_constant_beta_recency_closed_form():
    L, H, T = 2, 3, 40
    beta = np.full((L, H, T), 0.9, np.float32)
    M = 100
    keep = dbtrim.keep_mask(dbtrim.log_retention(beta, T), M)
    per = M // (L * H)                 # 16 most recent positions per head
    extra = M - per * L * H            # the next older position in the lowest (layer, head) heads
    for lh in range(L * H):
        want = np.zeros(T, bool)
        want[T - per:] = True
        if lh < extra:
            want[T - per - 1] = True
        np.testing.assert_array_equal(keep.reshape(L * H, T)[lh], want)


def test_compaction_plan_by_brute_force():
    rng = np.random.default_rng(12)
    L, H, T, P = 2, 2, 64, 16
    keep = rng.random((L, H, T)) < 0.3
    pt = rng.permutation(L * H * (T // P)).reshape(L, H, T // P).astype(np.int32)
    src, lengths, offs, npg = dbtrim.compact_rows(keep, pt, P)
    assert lengths.sum() == keep.sum()
    assert np.all(npg == (lengths + P - 1) // P)
    dst = 0
    for l in range(L):
        for h in range(H):
            lh = l * H + h
            assert offs[lh] == dst
            pos = [i for i in range(T) if keep[l, h, i]]
            for j, i in enumerate(pos):
                assert src[offs[lh] * P + j] == pt[l, h, i // P] * P + i % P
            for j in range(len(pos), npg[lh] * P):
                assert src[offs[lh] * P + j] == -1
            dst += npg[lh]

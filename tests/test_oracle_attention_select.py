"""Pins for the oracle's attention, window mass and selection routines (CPU only).

Attention is checked against pure-Python loops (math.exp, math.fsum) on tiny inputs and against closed forms;
selection against Python's own sorted() with an explicit (score desc, index asc) key.
"""
import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import attention, select


def loop_attention(q, K, V):
    G, D = q.shape
    n = K.shape[0]
    p = np.zeros((G, n))
    o = np.zeros((G, D))
    for h in range(G):
        s = [sum(float(q[h, d]) * float(K[i, d]) for d in range(D)) / math.sqrt(D) for i in range(n)]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        tot = math.fsum(e)
        for i in range(n):
            p[h, i] = e[i] / tot
        for d in range(D):
            o[h, d] = math.fsum(p[h, i] * float(V[i, d]) for i in range(n))
    return p, o


@settings(max_examples=40, deadline=None)
@given(st.integers(0, 2 ** 31 - 1), st.integers(1, 4), st.integers(1, 9), st.sampled_from([2, 4, 8]))
def test_attention_matches_loops(seed, G, n, D):
    rng = np.random.default_rng(seed)
    q, K, V = rng.standard_normal((G, D)) * 2, rng.standard_normal((n, D)), rng.standard_normal((n, D))
    _, p, o = attention.gqa_decode(q, K, V)
    p2, o2 = loop_attention(q, K, V)
    np.testing.assert_allclose(p, p2, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)


def test_zero_keys_give_uniform_weights_and_mean_value():
    rng = np.random.default_rng(5)
    n = 37
    q = rng.standard_normal((4, 128))
    K = np.zeros((n, 128))
    V = rng.standard_normal((n, 128))
    _, p, o = attention.gqa_decode(q, K, V)
    assert np.all(p == 1.0 / n)
    np.testing.assert_allclose(o, np.broadcast_to(V.mean(axis=0), o.shape), rtol=1e-13, atol=1e-14)


def test_dominant_key_returns_its_value():
    rng = np.random.default_rng(6)
    q = np.ones((2, 128))
    K = rng.standard_normal((50, 128)) * 0.01
    K[17] = 50.0 * math.sqrt(128) / 128  # logit +50 against ~0
    V = rng.standard_normal((50, 128))
    _, p, o = attention.gqa_decode(q, K, V)
    # every other weight is below exp(-49): o equals v_17 to far below fp64 resolution of |v| ~ 1
    assert np.max(np.abs(o - V[17])) < 1e-15
    assert np.all(p[:, 17] > 1 - 1e-15)


def test_window_mass_brute_force_and_conservation():
    rng = np.random.default_rng(7)
    G, n_win, W, tail = 4, 6, 8, 5
    p = rng.random((G, n_win * W + tail))
    p /= p.sum(axis=1, keepdims=True)
    kw = np.concatenate([np.repeat(rng.permutation(n_win), W), -np.ones(tail, np.int64)])
    mass = attention.window_mass(p, kw, n_win)
    for w in range(n_win):
        ref = math.fsum(p[h, i] for h in range(G) for i in range(p.shape[1]) if kw[i] == w) / G
        assert abs(mass[w] - ref) < 1e-15
    tail_mass = p[:, kw < 0].sum() / G
    assert abs(mass.sum() + tail_mass - 1.0) < 1e-12


score_lists = st.lists(st.sampled_from([0.0, -0.0, 1.0, 1.0, 2.5, 3.0, 1e-30, 7.0]), min_size=1, max_size=40)


@settings(max_examples=200, deadline=None)
@given(score_lists, st.integers(0, 45))
def test_topk_matches_sorted(scores, k):
    sc = np.array(scores)
    ref = sorted(range(len(scores)), key=lambda i: (-scores[i], i))[:k]
    assert list(select.topk(sc, k)) == ref


def test_nan_rejected():
    with pytest.raises(ValueError):
        select.rank_order(np.array([1.0, float("nan")]))


@settings(max_examples=100, deadline=None)
@given(st.lists(st.floats(0, 10, allow_nan=False), min_size=1, max_size=30), st.integers(0, 12),
       st.integers(0, 12), st.integers(0, 2 ** 31 - 1))
def test_three_tier_caps_and_permanence(scores, bf, bq, seed):
    rng = np.random.default_rng(seed)
    n = len(scores)
    tier = rng.choice([select.FULL, select.INT2, select.EVICTED], size=n).astype(np.int8)
    new = select.three_tier(np.array(scores), tier, bf, bq)
    res = [i for i in range(n) if tier[i] != select.EVICTED]
    order = sorted(res, key=lambda i: (-scores[i], i))
    for r, i in enumerate(order):
        want = select.FULL if r < bf else (select.INT2 if r < bf + bq else select.EVICTED)
        assert new[i] == want
    assert np.all(new[tier == select.EVICTED] == select.EVICTED)
    assert (new == select.FULL).sum() == min(bf, len(res))
    assert (new == select.INT2).sum() == min(bq, max(0, len(res) - bf))


def test_three_tier_strictly_decreasing_is_a_prefix_split():
    n = 20
    sc = np.arange(n, 0, -1).astype(float)
    new = select.three_tier(sc, np.zeros(n, np.int8), 5, 7)
    np.testing.assert_array_equal(new, [0] * 5 + [1] * 7 + [2] * 8)


def brute_two_stage(a, s2, b, alpha):
    b1 = math.floor(alpha * b)
    i1 = sorted(range(len(a)), key=lambda i: (-a[i], i))[:b1]
    rest = [i for i in sorted(range(len(a)), key=lambda i: (-s2[i], i)) if i not in i1]
    return sorted(i1 + rest[:b - b1])


@settings(max_examples=100, deadline=None)
@given(st.integers(0, 2 ** 31 - 1), st.integers(1, 40), st.sampled_from([0.0, 0.25, 0.5, 1.0]))
def test_two_stage_matches_brute_force(seed, n, alpha):
    rng = np.random.default_rng(seed)
    a = np.round(rng.random(n), 1)
    s2 = np.round(rng.random(n), 1)
    b = int(rng.integers(0, n + 1))
    assert list(select.two_stage(a, s2, b, alpha)) == brute_two_stage(list(a), list(s2), b, alpha)


def test_two_stage_special_cases():
    rng = np.random.default_rng(8)
    a = rng.random(100)
    n = rng.random(100)
    # alpha = 1: pure top-b by A
    np.testing.assert_array_equal(select.two_stage(a, a * n, 30, 1.0), np.sort(select.topk(a, 30)))
    # constant projected norm: S2 is proportional to A, so the selection is top-b by A
    np.testing.assert_array_equal(select.two_stage(a, a * 3.0, 30, 0.5), np.sort(select.topk(a, 30)))


@settings(max_examples=60, deadline=None)
@given(st.integers(0, 2 ** 31 - 1), st.integers(1, 200))
def test_global_topm_matches_sorted(seed, n):
    rng = np.random.default_rng(seed)
    sc = np.round(rng.standard_normal(n), 1)
    m = int(rng.integers(0, n + 1))
    keep = select.global_topm(sc, m)
    ref = set(sorted(range(n), key=lambda i: (-sc[i], i))[:m])
    assert set(np.flatnonzero(keep)) == ref

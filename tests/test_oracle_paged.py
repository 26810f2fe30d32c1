"""Pins for the oracle's decode attention over a per-head paged cache (CPU only)."""
import math

import numpy as np

from oracle import dbtrim, paged


def _scatter(rng, seq, page, n_pool):
    """Scatter a contiguous sequence [n][D] into a pool of n_pool pages at random distinct page ids; returns the
    pool and the page list (the pool's other rows hold noise that must never be read)."""
    n, D = seq.shape
    n_pages = -(-n // page)
    ids = rng.choice(n_pool, n_pages, replace=False)
    pool = rng.standard_normal((n_pool, page, D)) * 100.0
    for j, pid in enumerate(ids):
        rows = seq[j * page:(j + 1) * page]
        pool[pid, :rows.shape[0]] = rows
    return pool, ids.astype(np.int32)


def test_paged_equals_attention_over_the_contiguous_sequence():
    rng = np.random.default_rng(31)
    for n, page in ((1, 16), (15, 16), (16, 16), (17, 16), (100, 16), (64, 32), (77, 32)):
        G, D = 4, 8
        q = rng.standard_normal((G, D))
        K = rng.standard_normal((n, D))
        V = rng.standard_normal((n, D))
        kp, ids = _scatter(rng, K, page, 40)
        vp = np.zeros_like(kp)
        for j, pid in enumerate(ids):
            rows = V[j * page:(j + 1) * page]
            vp[pid, :rows.shape[0]] = rows
        o = paged.paged_gqa_decode(q, kp, vp, ids, n, page)
        # textbook attention by loops on the contiguous arrays
        for h in range(G):
            s = [math.fsum(q[h, d] * K[i, d] for d in range(D)) / math.sqrt(D) for i in range(n)]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            tot = math.fsum(e)
            ref = [math.fsum(e[i] * V[i, d] for i in range(n)) / tot for d in range(D)]
            np.testing.assert_allclose(o[h], ref, rtol=1e-12, atol=1e-12)


def test_rows_past_the_length_are_never_keys():
    rng = np.random.default_rng(32)
    q = rng.standard_normal((2, 8))
    kp = rng.standard_normal((3, 16, 8))
    vp = rng.standard_normal((3, 16, 8))
    ids = np.array([2, 0], np.int32)
    o1 = paged.paged_gqa_decode(q, kp, vp, ids, 20, 16)
    kp2, vp2 = kp.copy(), vp.copy()
    kp2[0, 4:] = 1e6   # rows 4.. of the second listed page lie past the length
    vp2[0, 4:] = -1e6
    kp2[1] = 1e6       # an unlisted page
    o2 = paged.paged_gqa_decode(q, kp2, vp2, ids, 20, 16)
    np.testing.assert_array_equal(o1, o2)


def test_identical_keys_give_the_mean_value_and_empty_rows_zeros():
    rng = np.random.default_rng(33)
    q = rng.standard_normal((4, 8))
    kp = np.tile(rng.standard_normal(8), (5, 16, 1))
    vp = rng.standard_normal((5, 16, 8))
    ids = np.array([3, 1, 4], np.int32)
    o = paged.paged_gqa_decode(q, kp, vp, ids, 40, 16)
    mean = (vp[3].sum(0) + vp[1].sum(0) + vp[4, :8].sum(0)) / 40.0
    np.testing.assert_allclose(o, np.tile(mean, (4, 1)), rtol=1e-12, atol=1e-12)
    assert not paged.paged_gqa_decode(q, kp, vp, ids, 0, 16).any()


def test_paged_over_the_compaction_output_equals_attention_over_kept_positions():
    rng = np.random.default_rng(34)
    L, H, T, page, D = 1, 2, 64, 16, 8
    keep = rng.random((L, H, T)) < 0.4
    page_table = rng.permutation(L * H * T // page).reshape(L * H, T // page).astype(np.int32)
    k_src = rng.standard_normal((L * H * T // page, page, D))
    v_src = rng.standard_normal((L * H * T // page, page, D))
    src, lengths, page_offset, n_pages = dbtrim.compact_rows(keep, page_table, page)
    k_out = np.zeros((int(n_pages.sum()) * page, D))
    v_out = np.zeros_like(k_out)
    ok = src >= 0
    k_out[ok] = k_src.reshape(-1, D)[src[ok]]
    v_out[ok] = v_src.reshape(-1, D)[src[ok]]
    k_out = k_out.reshape(-1, page, D)
    v_out = v_out.reshape(-1, page, D)
    for r in range(L * H):
        q = rng.standard_normal((4, D))
        ids = page_offset[r] + np.arange(n_pages[r])
        o = paged.paged_gqa_decode(q, k_out, v_out, ids, int(lengths[r]), page)
        pos = np.flatnonzero(keep.reshape(L * H, T)[r])
        rows = page_table[r][pos // page] * page + pos % page
        K = k_src.reshape(-1, D)[rows]
        V = v_src.reshape(-1, D)[rows]
        s = q @ K.T / math.sqrt(D)
        p = np.exp(s - s.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        np.testing.assert_allclose(o, p @ V, rtol=1e-12, atol=1e-12)

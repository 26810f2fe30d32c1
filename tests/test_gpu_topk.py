"""GPU parity of the generic budgeted top-k (kvc_topk) against the oracle's selection (needs an MI355X): bit-exact
index sets (ascending) on the same fp32 scores, over lengths that are and are not multiples of 16, k from 0 to n,
and score distributions with many ties, constants, negatives and attention-like mass."""
import sys

import numpy as np
import pytest
import torch

from kv_cache_compression_gqa_amd import selection
from oracle import select as osel

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _cases(rng, n):
    yield "normal", rng.standard_normal(n)
    yield "ties", np.round(rng.standard_normal(n), 1)
    yield "constant", np.full(n, 0.25)
    yield "negative", -np.abs(rng.standard_normal(n)) * 1e3
    e = np.exp(rng.standard_normal(n) * 3.0)
    yield "attention", e / e.sum()


@pytest.mark.parametrize("n", [1, 15, 16, 17, 1000, 4097, 65539])
def test_topk_matches_oracle(gpu_lib, n):
    rng = np.random.default_rng(n)
    for name, sc in _cases(rng, n):
        s32 = sc.astype(np.float32)
        dev = torch.from_numpy(s32).cuda()
        for k in sorted({0, 1, n // 3, n // 2, n - 1, n} - {-1}):
            if k < 0 or k > n:
                continue
            got = selection.topk(dev, k).cpu().numpy()
            want = np.sort(osel.topk(s32.astype(np.float64), k))
            assert np.array_equal(got, want), f"n={n} {name} k={k}"
    log(f"topk n={n}: every case matches")


def test_topk_large(gpu_lib):
    """4 M entries with heavy ties, k = 10%."""
    rng = np.random.default_rng(99)
    n = (1 << 22) + 5
    s32 = np.round(rng.standard_normal(n), 2).astype(np.float32)
    k = n // 10
    got = selection.topk(torch.from_numpy(s32).cuda(), k).cpu().numpy()
    want = np.sort(osel.topk(s32.astype(np.float64), k))
    assert np.array_equal(got, want)


def test_topk_nan_and_infinite_scores_give_indices_in_range(gpu_lib):
    """A NaN leaves the order undefined, but the output is still k distinct ascending indices in [0, n), whatever
    the length (no padded entry can be chosen); -inf and -FLT_MAX rank last among finite scores."""
    rng = np.random.default_rng(7)
    for n in (17, 1000, 8195):
        s32 = rng.standard_normal(n).astype(np.float32)
        s32[:3] = [np.float32(-np.inf), np.float32(-3.4028235e38), np.float32(-np.inf)]
        for k in (n - 1, n):
            got = selection.topk(torch.from_numpy(s32).cuda(), k).cpu().numpy()
            want = np.sort(osel.topk(s32.astype(np.float64), k))
            assert np.array_equal(got, want), (n, k)
        bad = s32.copy()
        bad[5] = np.float32("nan")
        bad[6] = -np.float32("nan")
        for k in (1, n // 2, n - 1, n):
            got = selection.topk(torch.from_numpy(bad).cuda(), k).cpu().numpy()
            assert got.size == k and np.all(np.diff(got) > 0) and got.min() >= 0 and got.max() < n, (n, k)


def test_topk_misleading_sample_takes_the_fallback(gpu_lib):
    """The entries the engine samples (its documented rule, tests.engine_sampling.sampled_entries) hold the highest
    scores, so the sampled window lies far above the k-th key; the fallback classification still gives the exact
    top-k, here with a ragged length."""
    from tests.engine_sampling import sampled_entries
    rng = np.random.default_rng(5)
    n = (1 << 20) + 3
    s32 = rng.standard_normal(n).astype(np.float32)
    s32[sampled_entries(n)] = np.float32(1e6)
    for k in (n // 10, n // 2):
        got = selection.topk(torch.from_numpy(s32).cuda(), k).cpu().numpy()
        want = np.sort(osel.topk(s32.astype(np.float64), k))
        assert np.array_equal(got, want), k


def test_topk_fallback_over_many_workgroups(gpu_lib):
    """The fallback classification at 2^24 + 5 entries: with a misleading sample, every one of the 33 candidate
    workgroups reclassifies its own 256 chunks (the last one ragged) before the candidate passes."""
    from tests.engine_sampling import sampled_entries
    rng = np.random.default_rng(21)
    n = (1 << 24) + 5
    s32 = np.round(rng.standard_normal(n), 3).astype(np.float32)
    s32[sampled_entries(n)] = np.float32(1e6)
    k = n // 10
    log(f"topk fallback n={n} k={k}")
    got = selection.topk(torch.from_numpy(s32).cuda(), k).cpu().numpy()
    want = np.sort(osel.topk(s32.astype(np.float64), k))
    assert np.array_equal(got, want)


def test_topk_zeros_and_denormals_rank_by_value(gpu_lib):
    """+0 and -0 tie (ranked by index); the smallest positive and negative subnormals rank on either side of them."""
    tiny = np.float32(1.4e-45)
    base = np.array([0.0, -0.0, tiny, -tiny, 2 * tiny, -2 * tiny, 1e-38, -1e-38, 1.0, -1.0], np.float32)
    s32 = np.tile(base, 3000)
    np.random.default_rng(3).shuffle(s32)
    n = s32.size
    for k in (1, 3000, 6000, 9000, 12000, 15000, n - 1):
        got = selection.topk(torch.from_numpy(s32).cuda(), k).cpu().numpy()
        want = np.sort(osel.topk(s32.astype(np.float64), k))
        assert np.array_equal(got, want), k

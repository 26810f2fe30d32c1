"""GPU parity of the CriticalKV scores (observation-window attention A, projected-value norm N, group means A_g and
S2_g) and of the two-stage selection against the CPU oracle, through the C ABI.

Bars: A, N, A_g, S2_g within 2e-3 relative of the fp64 oracle (N and S2 on sampled tokens at the full 64K shape,
where the oracle's 1.1 TFLOP product is out of reach); selected index sets bit-exact against the oracle's
two-stage selection fed the GPU's fp32 scores."""
import dataclasses

import numpy as np
import pytest

from kv_cache_compression_gqa_amd import abi, configs, synth
from oracle import criticalkv as ock
from oracle import fp as ofp
from oracle import select as osel
from tests.decode_parity import rel_check

pytestmark = pytest.mark.gpu

RTOL = 2e-3


def _gpu_scores(inp, dtype):
    import torch
    from kv_cache_compression_gqa_amd import criticalkv
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    t = {name: torch.from_numpy(getattr(inp, name).view(np.int16)).cuda().view(tdt)
         for name in ("q_obs", "k", "v", "w_o")}
    out = criticalkv.scores(t["q_obs"], t["k"], t["v"], t["w_o"], abi.KVC_BF16 if dtype == "bf16" else abi.KVC_F16)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items() if not k.startswith("_")}


def _oracle_inputs(inp, dtype):
    f = lambda x: ofp.storage_to_f64(x, dtype)  # noqa: E731
    return f(inp.q_obs), f(inp.k), f(inp.v), f(inp.w_o)


def _check_selection(a_g, s2_g, budget, alpha):
    import torch
    from kv_cache_compression_gqa_amd import criticalkv
    idx = criticalkv.two_stage(torch.from_numpy(a_g).cuda(), torch.from_numpy(s2_g).cuda(), budget, alpha)
    torch.cuda.synchronize()
    ref = ock.select(a_g.astype(np.float64), s2_g.astype(np.float64), budget, alpha)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref)


@pytest.mark.parametrize("dtype,hq,hkv,n", [("bf16", 8, 2, 1000), ("f16", 8, 2, 777), ("bf16", 8, 1, 2080),
                                            ("bf16", 2, 2, 530)])
def test_criticalkv_scores_small(gpu_lib, dtype, hq, hkv, n):
    cfg = dataclasses.replace(configs.CRITICALKV_64K, hq=hq, hkv=hkv, dtype=dtype, budget=64)
    inp = synth.make_criticalkv(cfg, n_keys=n, d_model=256, n_salient=12)
    g = _gpu_scores(inp, dtype)
    q, k, v, w = _oracle_inputs(inp, dtype)
    A, N, A_g, S2_g = ock.scores(q, k, v, w, cfg.group)
    rel_check("A", g["a_head"], A, rtol=RTOL)
    rel_check("N", g["norm"], N, rtol=RTOL)
    rel_check("A_g", g["a_group"], A_g, rtol=RTOL)
    rel_check("S2_g", g["s2_group"], S2_g, rtol=RTOL)
    # each observation row's probabilities sum to 1, so every head's A sums to 1
    np.testing.assert_allclose(g["a_head"].astype(np.float64).sum(axis=1), 1.0, rtol=1e-4)
    _check_selection(g["a_group"], g["s2_group"], cfg.budget, cfg.alpha)


def test_criticalkv_full_size(gpu_lib):
    """65536 keys, 32/8 heads, d_model 4096: A over every key; N and S2 on 512 sampled keys; full selection."""
    cfg = configs.CRITICALKV_64K
    print(f"full-size CriticalKV: n={cfg.n_keys} hq={cfg.hq} hkv={cfg.hkv} d_model={cfg.d_model}", flush=True)
    inp = synth.make_criticalkv(cfg)
    g = _gpu_scores(inp, cfg.dtype)
    q, k, v, w = _oracle_inputs(inp, cfg.dtype)
    rows = np.sort(np.random.default_rng(3).choice(cfg.n_keys, 512, replace=False))
    rows[0] = 0          # the sink
    rows[-1] = cfg.n_keys - 1
    A, N, A_g, S2_g = ock.scores(q, k, v, w, cfg.group, rows=rows)
    rel_check("A", g["a_head"], A, rtol=RTOL)
    rel_check("A_g", g["a_group"], A_g, rtol=RTOL)
    rel_check("N (sampled)", g["norm"][:, rows], N, rtol=RTOL)
    rel_check("S2_g (sampled)", g["s2_group"][:, rows], S2_g, rtol=RTOL)
    _check_selection(g["a_group"], g["s2_group"], cfg.budget, cfg.alpha)


@pytest.mark.parametrize("budget,alpha", [(2048, 0.5), (2048, 1.0), (2048, 0.0), (1, 0.5), (4096, 0.25)])
def test_two_stage_ties_and_edges(gpu_lib, budget, alpha):
    """Scores on a coarse grid (many exact ties across threads); stage cuts fall inside tie groups."""
    rng = np.random.default_rng(budget + int(alpha * 100))
    a = (np.round(rng.standard_normal((3, 65536)) * 4.0) / 4.0).astype(np.float32)
    s2 = (np.round(rng.standard_normal((3, 65536)) * 2.0) / 2.0).astype(np.float32)
    a[1, :1000] = 0.0
    a[1, 1000:1500] = -0.0
    _check_selection(a, s2, budget, alpha)


def test_two_stage_constant_rows_and_degenerate_budgets(gpu_lib):
    """Rows whose every entry is equal (all 65536 in one histogram bin: more candidates than the LDS path holds, so
    they are ranked from global memory; the order is then the index order), stage 1 from LDS with stage 2 from
    global memory, a row of one entry, stage budgets of 0 and of everything, odd lengths."""
    rng = np.random.default_rng(41)
    a = np.full((2, 65536), 0.25, np.float32)
    s2 = np.full((2, 65536), -1.5, np.float32)
    s2[1, ::7] = 3.0
    for budget, alpha in ((2048, 0.5), (65536, 0.5), (5000, 0.0), (5000, 1.0), (1, 1.0)):
        _check_selection(a, s2, budget, alpha)
    # stage 1 resolved from LDS, stage 2 (every second score equal) from global memory
    a = rng.standard_normal((2, 65536)).astype(np.float32)
    s2 = np.full((2, 65536), -1.5, np.float32)
    _check_selection(a, s2, 2048, 0.5)
    one = np.array([[0.5]], np.float32)
    _check_selection(one, one, 1, 0.5)
    _check_selection(one, one, 1, 0.0)
    a = rng.standard_normal((3, 4097)).astype(np.float32)
    s2 = rng.standard_normal((3, 4097)).astype(np.float32)
    for budget, alpha in ((4097, 0.3), (4096, 0.0), (100, 1.0), (2049, 0.5)):
        _check_selection(a, s2, budget, alpha)


def test_two_stage_small_rows(gpu_lib):
    rng = np.random.default_rng(5)
    a = rng.standard_normal((5, 300)).astype(np.float32)
    s2 = rng.standard_normal((5, 300)).astype(np.float32)
    _check_selection(a, s2, 100, 0.5)
    _check_selection(a, s2, 300, 0.5)

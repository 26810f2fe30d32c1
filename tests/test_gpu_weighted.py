"""GPU parity of the window score weighted by per-position, per-head weights (CriticalKV's projected-value norm
plugged into QEvict's cumulative window score) against the oracle (needs an MI355X).

Tolerances as for the plain decode: weighted window mass and cumulative score |g - r| <= 2e-3 |r| + 1e-12, outputs
per head row within 2e-3 max|r|, tiers and plan lists bit-exact when the oracle's router is fed the GPU's scores.
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

from kv_cache_compression_gqa_amd import abi, configs, criticalkv, synth
from oracle import criticalkv as ockv
from oracle.fp import storage_to_f64
from tests.decode_parity import run_decode_parity

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_weighted_score_matches_oracle(gpu_lib, dtype):
    log(f"case: weighted window score, tiny workload, {dtype}, log-normal weights")
    cfg = dataclasses.replace(configs.TINY, dtype=dtype)
    inp = synth.make_decode(cfg, steps=12)
    U, NW = len(inp.units), inp.n_windows_max
    G = cfg.hq // cfg.hkv
    w = np.random.default_rng(11).lognormal(size=(U, G, NW * cfg.window + 64))  # a stride past NW * W
    run_decode_parity(cfg, inp=inp, token_weight=torch.from_numpy(w.astype(np.float32)).cuda(),
                      oracle_weight=w.astype(np.float32).astype(np.float64), log=log)


def test_weighted_score_2k_context_g8(gpu_lib):
    log("case: weighted window score, 8 units at 2048 tokens, G = 8")
    cfg = dataclasses.replace(configs.LLAMA3_8B_LAYER_32K, name="ctx2k_g8", hq=64, context=2048 + 17, steps=8,
                              route_every=4)
    inp = synth.make_decode(cfg)
    U, NW = len(inp.units), inp.n_windows_max
    w = np.random.default_rng(12).lognormal(size=(U, 8, NW * cfg.window)).astype(np.float32)
    run_decode_parity(cfg, inp=inp, token_weight=torch.from_numpy(w).cuda(), oracle_weight=w.astype(np.float64),
                      probs=False, log=log)


def test_weighted_score_many_units(gpu_lib):
    """1280 units at G = 4 (bf16): the many-round launch shape, whose INT2 tasks take two windows each, with the
    weights loaded beside each task's other loads; units spread over layers, sequences and heads."""
    cfg = dataclasses.replace(configs.TINY, name="many_weighted", seed=15, hq=16, hkv=4, dtype="bf16", layers=32,
                              batch=10, context=640, n_salient=5, budget_full=4, budget_int2=7, steps=4, route_every=2)
    inp, plan = synth.make_decode_shared_layers(cfg)
    U, NW = cfg.n_units, inp.n_windows_max
    w = np.random.default_rng(13).lognormal(size=(U, 4, NW * cfg.window)).astype(np.float32)
    log(f"case: weighted window score, {U} units, G = 4")
    run_decode_parity(cfg, inp=inp, plan=plan, check_units=[0, 333, 777, U - 1],
                      token_weight=torch.from_numpy(w).cuda(), oracle_weight=w.astype(np.float64), log=log)


def test_criticalkv_norms_weight_the_window_score(gpu_lib):
    """End to end: the GPU's |V W_O,h|_1 (kvc_score(CRITICALKV) over the tiny cache's prefill keys and values, a
    seeded W_O) weights the decode's window score; the oracle computes its own norms from the same inputs."""
    cfg = configs.TINY
    log("case: CriticalKV norms from the GPU weight the tiny decode's window score")
    inp = synth.make_decode(cfg, steps=8)
    U, NW, W, D = len(inp.units), inp.n_windows_max, cfg.window, cfg.head_dim
    G = cfg.hq // cfg.hkv
    n = NW * W
    assert U == cfg.hkv and int(inp.tail0.max()) == 0
    k = inp.k_win.reshape(U, n, D)
    v = inp.v_win.reshape(U, n, D)
    rng = np.random.default_rng(13)
    q_obs = synth.to_storage_bits(rng.standard_normal((cfg.hq, 32, D)), cfg.dtype)
    dm = cfg.hq * D
    w_o = synth.to_storage_bits(rng.standard_normal((cfg.hq * D, dm)) / np.sqrt(dm), cfg.dtype)
    dt = torch.float16 if cfg.dtype == "f16" else torch.bfloat16
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(dt)  # noqa: E731
    out = criticalkv.scores(dev(q_obs), dev(k), dev(v), dev(w_o), abi.KVC_F16 if cfg.dtype == "f16" else abi.KVC_BF16)
    torch.cuda.synchronize()
    norm = out["norm"].view(U, G, n)
    wo64 = storage_to_f64(w_o, cfg.dtype)
    ref = np.zeros((U, G, n))
    for g in range(U):
        vg = storage_to_f64(v[g], cfg.dtype)
        for h in range(G):
            ref[g, h] = ockv.projected_value_l1(vg, wo64[(g * G + h) * D:(g * G + h + 1) * D])
    got = norm.cpu().numpy()
    assert np.all(np.abs(got - ref) <= 2e-3 * np.abs(ref) + 1e-12)
    run_decode_parity(cfg, inp=inp, token_weight=norm, oracle_weight=ref, log=log)


def test_weighted_score_llama_layer_32k(gpu_lib):
    """The 32K layer at full size with log-normal per-position weights in the window score, through the first
    routing event; the oracle follows units 0 and 5."""
    cfg = dataclasses.replace(configs.LLAMA3_8B_LAYER_32K, steps=20)
    log("case: weighted window score, llama3_8b_layer_ctx32k_bf16, 20 steps, oracle on units 0 and 5")
    inp = synth.make_decode(cfg)
    U, NW = len(inp.units), inp.n_windows_max
    G = cfg.hq // cfg.hkv
    w = np.random.default_rng(23).lognormal(size=(U, G, NW * cfg.window)).astype(np.float32)
    run_decode_parity(cfg, inp=inp, token_weight=torch.from_numpy(w).cuda(), oracle_weight=w.astype(np.float64),
                      check_units=[0, 5], check_steps=[0, 15, 16, 19], probs=False, log=log)

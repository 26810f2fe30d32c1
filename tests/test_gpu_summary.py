"""GPU parity of the span-summary term (SEKV's mixed-resolution attention, untrained reading): every evicted window
leaves the means of its keys and values, attended after the tail with a ln 32 size correction (needs an MI355X).

Bars: summaries byte-exact (both sides round the exact mean to fp32 and then to the storage dtype); outputs, window
masses and cumulative scores as for the plain decode (2e-3); tiers and lists bit-exact on the GPU's scores.
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

from kv_cache_compression_gqa_amd import abi, configs, synth
from kv_cache_compression_gqa_amd.session import DecodeSession
from tests.decode_parity import run_decode_parity

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_summaries_tiny(gpu_lib, dtype):
    log(f"case: span summaries, tiny workload, {dtype}, 12 steps")
    cfg = dataclasses.replace(configs.TINY, dtype=dtype)
    sess, oracles, _ = run_decode_parity(cfg, steps=12, probs=False, summaries=True, log=log)
    assert int(sess.n_sum.max().item()) == 16   # the first event evicts 16 windows per unit, later ones none


def test_summaries_2k_context_g8_and_g1(gpu_lib):
    for hq, hkv in ((64, 8), (8, 8)):
        cfg = dataclasses.replace(configs.LLAMA3_8B_LAYER_32K, name=f"ctx2k_g{hq // hkv}", hq=hq, hkv=hkv,
                                  context=2048 + 40, steps=12, route_every=4)
        log(f"case: span summaries, {cfg.name}, {hkv} units")
        run_decode_parity(cfg, probs=False, summaries=True, log=log)


@pytest.mark.parametrize("hkv, batch, dtype", [(2, 20, "f16"), (4, 10, "bf16")], ids=["g8_f16", "g4_bf16"])
def test_summaries_many_units(gpu_lib, hkv, batch, dtype):
    """1280 units (the many-round launch shape: two INT2 windows per task, 4-wave workgroups), G = 8 and 4."""
    cfg = dataclasses.replace(configs.TINY, name="many_sum", seed=14, hq=16, hkv=hkv, dtype=dtype, layers=32,
                              batch=batch, context=640, n_salient=5, budget_full=4, budget_int2=7, steps=4,
                              route_every=2)
    inp, plan = synth.make_decode_shared_layers(cfg)
    log(f"case: span summaries, {cfg.n_units} units, G = {16 // hkv}, {dtype}")
    run_decode_parity(cfg, inp=inp, plan=plan, check_units=[0, 333, 777, cfg.n_units - 1], probs=False,
                      summaries=True, log=log)


def test_summaries_reject_probabilities_and_over_capacity(gpu_lib):
    cfg = configs.TINY
    inp = synth.make_decode(cfg, steps=6)
    sess = DecodeSession(inp, summaries=True)
    for _ in range(4):
        sess.step()
    assert int(sess.h_sum.max()) > 0
    import ctypes as C
    pr = torch.zeros((sess.U, sess.G, sess.probs_stride()), dtype=torch.float32, device="cuda")
    args = sess.decode_args(sess.t, probs=pr)
    ws = sess.workspace(sess.decode_args(sess.t))
    L = abi.lib()
    st = L.kvc_decode_attn(C.byref(sess._cache), C.byref(args), abi.ptr(ws), ws.numel(), None)
    assert st == abi.KVC_E_UNSUPPORTED            # summaries are attended without probabilities only
    assert L.kvc_decode_attn_workspace(C.byref(sess._cache), C.byref(args)) == 0
    args = sess.decode_args(sess.t)
    args.max_summary = sess.SM + 32                # past the capacity
    st = L.kvc_decode_attn(C.byref(sess._cache), C.byref(args), abi.ptr(ws), ws.numel(), None)
    assert st == abi.KVC_E_BUDGET
    assert sess.device_status() == 0


def test_summaries_with_weighted_score_and_event_schedule(gpu_lib):
    """Every option of the step at once: span summaries, the weighted window score and the event-only schedule
    (the weighted + summary kernel instantiation), with a tail that grows past one 32-token block."""
    cfg = dataclasses.replace(configs.TINY, name="tiny_all", steps=40, route_every=8, context=1024 + 20)
    log("case: summaries + weighted score + event schedule, tiny workload, 40 steps")
    inp = synth.make_decode(cfg)
    U, NW = len(inp.units), inp.n_windows_max
    G = cfg.hq // cfg.hkv
    w = np.random.default_rng(21).lognormal(size=(U, G, NW * cfg.window)).astype(np.float32)
    run_decode_parity(cfg, inp=inp, token_weight=torch.from_numpy(w).cuda(), oracle_weight=w.astype(np.float64),
                      score_schedule="event", summaries=True, probs=False, log=log)


def test_summaries_llama_layer_32k(gpu_lib):
    """The 32K layer at full size (8 KV-head units, 1024 windows each) with span summaries, through its first
    routing event (513 summaries per unit) and four summary-attending steps; the oracle follows units 0 and 5."""
    cfg = dataclasses.replace(configs.LLAMA3_8B_LAYER_32K, steps=20)
    log("case: span summaries, llama3_8b_layer_ctx32k_bf16, 20 steps, oracle on units 0 and 5")
    sess, _, _ = run_decode_parity(cfg, check_units=[0, 5], check_steps=[0, 15, 16, 17, 19], probs=False,
                                summaries=True, log=log)
    assert int(sess.n_sum.min().item()) == 513

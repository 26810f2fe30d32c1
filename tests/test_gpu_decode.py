"""GPU parity of the windowed three-tier decode path against the oracle (needs an MI355X).

Covers: per-step attention output, per-key probabilities, window mass and cumulative score; routing tiers and
lists (bit-exact on the GPU's scores); write-once ledger bytes; promoted copies; adversarial quantiser groups;
adversarial routing scores (ties, zeros, signed zeros); the write-once violation flag; ledger lists over more units
than one launch serves, with ragged counts and bad ids; determinism.
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

from kv_cache_compression_gqa_amd import configs, synth
from kv_cache_compression_gqa_amd.session import DecodeSession
from oracle import select as osel
from tests.decode_parity import compare_route, make_oracles, run_decode_parity, slot_snapshot

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_tiny_run_matches_oracle(gpu_lib):
    log("case: tiny_gqa4_ctx1k_f16, 8 steps, route every 4")
    run_decode_parity(configs.TINY, log=log)


def test_tiny_bf16_run_matches_oracle(gpu_lib):
    cfg = dataclasses.replace(configs.TINY, dtype="bf16", name="tiny_bf16", seed=11)
    log("case: tiny bf16 variant, 8 steps")
    run_decode_parity(cfg, log=log)


def test_ragged_tail_and_odd_budgets(gpu_lib):
    # 3 KV heads x G=2, context 1000 (31 windows + 8-token tail), budgets 5 / 7, route every 3 steps
    cfg = dataclasses.replace(configs.TINY, name="ragged", seed=12, hq=6, hkv=3, context=1000, n_salient=9,
                              budget_full=5, budget_int2=7, steps=10, route_every=3)
    log("case: ragged tail (1000 tokens), G=2, budgets 5/7")
    run_decode_parity(cfg, log=log)


def test_group_of_eight_and_one(gpu_lib):
    for hq, hkv in ((16, 2), (2, 2)):
        cfg = dataclasses.replace(configs.TINY, name=f"g{hq // hkv}", seed=13, hq=hq, hkv=hkv, context=640,
                                  n_salient=5, budget_full=4, budget_int2=6, steps=6, route_every=2)
        log(f"case: G={hq // hkv}")
        run_decode_parity(cfg, log=log)


@pytest.mark.parametrize("case", ["no_budget", "full_budget", "context_below_one_window", "exactly_one_window"])
def test_degenerate_budgets_and_contexts(gpu_lib, case):
    """Budgets 0/0 (every window evicted at the first event, then the tail alone is attended), a FULL budget equal to
    the window count (nothing quantised or evicted), a context shorter than one window (no window at all: the tail
    alone, with routing over an empty set), and a context of exactly one window (empty prefill tail)."""
    base = dict(name=f"degenerate_{case}", seed=15, context=640, n_salient=5, steps=6, route_every=2)
    if case == "no_budget":
        base.update(budget_full=0, budget_int2=0)
    elif case == "full_budget":
        base.update(budget_full=20, budget_int2=0)
    elif case == "context_below_one_window":
        base.update(context=20, n_salient=1, budget_full=1, budget_int2=1)
    else:
        base.update(context=32, n_salient=1, budget_full=1, budget_int2=1)
    cfg = dataclasses.replace(configs.TINY, **base)
    log(f"case: {case}")
    run_decode_parity(cfg, log=log)


def test_many_units_two_int2_windows_per_task(gpu_lib):
    """1280 units: a step takes many rounds of workgroups, so the launch switches to two INT2 windows per wave
    task and 4-wave workgroups. G = 8 (f16), 1 (bf16), 2 (f16) and 4 (f16), probabilities on; the oracle follows units
    spread over layers, sequences and heads, two of them layers 0 and 9 of one (sequence, KV head), whose
    outputs must differ (every layer holds its windows in an order of its own and has its own step inputs)."""
    for hq, hkv, batch, dtype in ((16, 2, 20, "f16"), (4, 4, 10, "bf16"), (8, 4, 10, "f16"), (16, 4, 10, "f16")):
        cfg = dataclasses.replace(configs.TINY, name=f"many_g{hq // hkv}", seed=14, hq=hq, hkv=hkv, dtype=dtype,
                                  layers=32, batch=batch, context=640, n_salient=5, budget_full=4, budget_int2=7,
                                  steps=4, route_every=2)
        inp, plan = synth.make_decode_shared_layers(cfg)
        pair = [cfg.unit_index(0, 3, 1), cfg.unit_index(9, 3, 1)]
        log(f"case: {cfg.name}, {cfg.n_units} units, {dtype}")
        _, _, out = run_decode_parity(cfg, inp=inp, plan=plan,
                                      check_units=sorted(set([0, 333, 777, cfg.n_units - 1] + pair)), log=log)
        assert not np.allclose(out[pair[0]], out[pair[1]], rtol=1e-2, atol=0.0)


def test_llama_layer_32k_run_matches_oracle(gpu_lib):
    # every unit runs on the GPU in one launch; the oracle follows two units exactly through all 64 steps
    log("case: llama3_8b_layer_ctx32k_bf16, 64 steps, oracle on units 0 and 5")
    run_decode_parity(configs.LLAMA3_8B_LAYER_32K, check_units=[0, 5], log=log)


def _adversarial_rows(dtype, rng):
    rows = []
    rows.append(np.full(128, 0.375))                                     # constant groups
    rows.append(np.where(np.arange(128) % 2 == 0, -0.5, 1.0))            # two-valued
    k = rng.integers(0, 4, 128)
    k[::32], k[1::32] = 0, 3
    rows.append(-1.5 + 0.25 * k)                                         # exactly on the grid
    rows.append(rng.standard_normal(128) * 1e-5)                         # fp16-subnormal zeros/scales
    rows.append(rng.standard_normal(128) * 3000.0)                       # large magnitudes
    rows.append(np.concatenate([np.full(32, -0.0), np.full(32, 0.0), rng.standard_normal(64)]))
    rows.append(rng.uniform(-1, 1, 128) * 60000.0)                       # near the fp16 range
    base = np.stack(rows)
    out = np.concatenate([base, rng.standard_normal((32 - len(rows), 128))])
    return synth.to_storage_bits(out, dtype)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_quantise_and_promote_adversarial_groups(gpu_lib, dtype):
    cfg = dataclasses.replace(configs.TINY, dtype=dtype, name=f"adv_{dtype}", seed=14)
    inp = synth.make_decode(cfg, steps=2)
    rng = np.random.default_rng(15)
    for w in range(8, 16):
        inp.k_win[0, w] = _adversarial_rows(dtype, rng)
        inp.v_win[0, w] = _adversarial_rows(dtype, rng)
    sess = DecodeSession(inp)
    oracles = make_oracles(inp)
    nw = inp.n_windows_max
    # windows 0..7 FULL, 8..15 INT2 (first demotion: quantised), rest evicted
    sc = np.zeros((len(inp.units), nw), np.float32)
    sc[:, :16] = np.arange(16, 0, -1)
    scores = torch.from_numpy(sc).cuda()
    snap = slot_snapshot(sess)
    sess.route(scores=scores)
    torch.cuda.synchronize()
    compare_route(sess, oracles, sc.astype(np.float64), snap)
    # promote 8..15 back to FULL, demote 0..7 to INT2 (their first demotion)
    sc2 = np.zeros_like(sc)
    sc2[:, 8:16] = 10.0
    sc2[:, 0:8] = 5.0
    snap = slot_snapshot(sess)
    sess.route(scores=torch.from_numpy(sc2).cuda())
    torch.cuda.synchronize()
    compare_route(sess, oracles, sc2.astype(np.float64), snap)
    assert sess.device_status() == 0


def test_route_adversarial_scores(gpu_lib):
    cfg = dataclasses.replace(configs.TINY, name="route_adv", seed=16)
    inp = synth.make_decode(cfg, steps=1)
    rng = np.random.default_rng(17)
    cases = [np.zeros(32), np.full(32, 1.0), np.where(np.arange(32) % 2 == 0, -0.0, 0.0),
             np.round(rng.random(32), 1), np.arange(32, dtype=float), np.arange(32, 0, -1, dtype=float),
             np.where(rng.random(32) < 0.5, 1e-30, 1e30)]
    for case in cases:
        for bf, bq in ((8, 8), (0, 5), (5, 0), (0, 0), (32, 0), (20, 20), (3, 40)):
            sess = DecodeSession(inp, budgets=(np.full(2, bf), np.full(2, bq)))
            oracles = make_oracles(inp)
            sc = np.stack([case, case[::-1]]).astype(np.float32)
            snap = slot_snapshot(sess)
            sess.route(scores=torch.from_numpy(sc).cuda())
            torch.cuda.synchronize()
            compare_route(sess, oracles, sc.astype(np.float64), snap)
    log("route: 49 adversarial cases match")


def test_write_once_violation_is_refused(gpu_lib):
    """A second quantisation of a window that already has its ledger copy is skipped and reported, even after
    every full-precision slot has been scribbled over: the ledger pool keeps its bytes."""
    inp = synth.make_decode(configs.TINY, steps=1)
    sess = DecodeSession(inp)
    sc = np.zeros((2, 32), np.float32)
    sc[:, :16] = np.arange(16, 0, -1)
    sess.route(scores=torch.from_numpy(sc).cuda())
    torch.cuda.synchronize()
    assert sess.device_status() == 0
    before = (sess.k_codes.clone(), sess.k_meta.clone(), sess.v_codes.clone(), sess.v_meta.clone())
    sess.k_full.fill_(123)
    sess.v_full.fill_(123)
    lst = torch.zeros((2, 32), dtype=torch.int32, device="cuda")
    lst[0, 0] = 10   # an INT2 window since the event
    cnt = torch.tensor([1, 0], dtype=torch.int32, device="cuda")
    import ctypes as C
    from kv_cache_compression_gqa_amd import abi
    abi.check(abi.lib().kvc_quantize_int2(C.byref(sess._cache), abi.ptr(lst), abi.ptr(cnt), 32, 1,
                                          abi.stream_handle()), "quantize")
    torch.cuda.synchronize()
    assert sess.device_status() == abi.KVC_DEV_LEDGER_REWRITE
    for a, b in zip(before, (sess.k_codes, sess.k_meta, sess.v_codes, sess.v_meta)):
        assert torch.equal(a, b)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_ledger_lists_over_more_units_than_one_launch_span(gpu_lib, dtype):
    """kvc_quantize_int2, then kvc_promote, on per-unit lists over 4100 units (the library serves at most 4096
    units per launch), with ragged counts (0 to 8 windows, one unit listing every window, one empty list) and
    out-of-range ids, every unit's windows at shuffled full-precision and ledger slots: codes, scale/zero words,
    ledger flags and promoted copies are byte-exact against the oracle quantiser at the windows' slots on sampled
    units on both sides of the span boundary, unlisted slots stay untouched, and the bad ids set the bound bit."""
    import ctypes as C
    from kv_cache_compression_gqa_amd import abi, layout
    from oracle.fp import f32_to_storage_rne
    from oracle.int2 import dequantize, quantize
    cfg = dataclasses.replace(configs.TINY, dtype=dtype, name=f"ledger_span_{dtype}", seed=24)
    inp = synth.make_decode(cfg, steps=1)
    U = 4100
    umap = np.arange(U) % len(inp.units)
    sess = DecodeSession(inp, unit_map=umap, budgets=(np.full(U, 16), np.full(U, 16)))
    NW = sess.NW
    assert sess.FS == NW and sess.LS == NW
    rng = np.random.default_rng(25)
    # shuffled slots: window w of unit u sits in full-precision slot fperm[u, w] and gets ledger slot lperm[u, w]
    fperm = np.stack([rng.permutation(NW) for _ in range(U)]).astype(np.int64)
    lperm = np.stack([rng.permutation(NW) for _ in range(U)]).astype(np.int64)
    uidx = torch.arange(U, device="cuda")[:, None]
    ft = torch.from_numpy(fperm).cuda()
    for pool in (sess.k_full, sess.v_full):
        orig = pool.clone()
        pool[uidx, ft] = orig
    sess.full_slot.copy_(ft.to(torch.int32))
    sess.ledger_slot.copy_(torch.from_numpy(lperm).cuda().to(torch.int32))
    counts = rng.integers(0, 9, U)
    counts[[3, 4097]] = NW
    counts[[10, 4096]] = (0, 5)
    lists = np.zeros((U, NW), np.int32)
    for u in range(U):
        lists[u, :counts[u]] = np.sort(rng.choice(NW, counts[u], replace=False))
    bad = {(3, 0): NW + 3, (4096, 2): -1}
    valid = lists.copy()
    for (u, j), w in bad.items():
        lists[u, j] = w
    lst = torch.from_numpy(lists).cuda()
    cnt = torch.from_numpy(counts.astype(np.int32)).cuda()
    L = abi.lib()
    log(f"case: quantise {int(counts.sum())} listed windows over {U} units ({dtype})")
    abi.check(L.kvc_quantize_int2(C.byref(sess._cache), abi.ptr(lst), abi.ptr(cnt), NW, int(counts.sum()),
                                  abi.stream_handle()), "quantize")
    torch.cuda.synchronize()
    assert sess.device_status() == abi.KVC_DEV_BOUND_EXCEEDED
    sample = [0, 1, 3, 10, 4095, 4096, 4097, 4099]
    sel = torch.tensor(sample, dtype=torch.int64, device="cuda")
    g = lambda t: t.index_select(0, sel).cpu().numpy()  # noqa: E731
    kc, vc = g(sess.k_codes), g(sess.v_codes).view(np.uint16)
    km, vm, led = g(sess.k_meta).view(np.uint32), g(sess.v_meta).view(np.uint32), g(sess.ledgered)
    expect = {}
    for r, u in enumerate(sample):
        b = int(umap[u])
        listed = {int(w) for j, w in enumerate(valid[u, :counts[u]]) if (u, j) not in bad}
        for w in range(NW):
            sl = int(lperm[u, w])
            if w not in listed:
                assert led[r, w] == 0 and not kc[r, sl].any() and not km[r, sl].any(), f"unit {u} window {w}"
                continue
            kq, ks, kz = quantize(inp.k_win[b, w], dtype)
            vq, vs, vz = quantize(inp.v_win[b, w], dtype)
            expect[(u, w)] = (kq, ks, kz, vq, vs, vz)
            assert led[r, w] == 1, f"ledger flag unit {u} window {w}"
            assert kc[r, sl].tobytes() == layout.k_codes_to_lib(kq).tobytes(), f"K codes unit {u} window {w}"
            assert vc[r, sl].tobytes() == layout.v_codes_to_lib(vq).tobytes(), f"V codes unit {u} window {w}"
            assert km[r, sl].tobytes() == layout.k_meta_to_lib(ks, kz).tobytes(), f"K meta unit {u} window {w}"
            assert vm[r, sl].tobytes() == layout.v_meta_to_lib(vs, vz).tobytes(), f"V meta unit {u} window {w}"
    # promotion of the same lists over scribbled full-precision slots
    sess.k_full.fill_(0x7E7E)
    sess.v_full.fill_(0x7E7E)
    log("case: promote the same lists")
    abi.check(L.kvc_promote(C.byref(sess._cache), abi.ptr(lst), abi.ptr(cnt), NW, int(counts.sum()),
                            abi.stream_handle()), "promote")
    torch.cuda.synchronize()
    assert sess.device_status() == abi.KVC_DEV_BOUND_EXCEEDED
    kw, vw = g(sess.k_full).view(np.uint16), g(sess.v_full).view(np.uint16)
    for r, u in enumerate(sample):
        for w in range(NW):
            sl = int(fperm[u, w])
            if (u, w) not in expect:
                assert np.all(kw[r, sl] == 0x7E7E) and np.all(vw[r, sl] == 0x7E7E), f"unit {u} window {w} written"
                continue
            kq, ks, kz, vq, vs, vz = expect[(u, w)]
            assert kw[r, sl].tobytes() == f32_to_storage_rne(dequantize(kq, ks, kz), dtype).tobytes(), (u, w)
            assert (layout.v_win_from_lib(vw[r, sl]).tobytes() ==
                    f32_to_storage_rne(dequantize(vq, vs, vz), dtype).tobytes()), (u, w)
    log(f"ledger lists over {U} units: {len(expect)} sampled windows match")


def test_probabilities_sum_to_one_and_runs_are_bitwise_reproducible(gpu_lib):
    results = []
    for _ in range(2):
        inp = synth.make_decode(configs.TINY)
        sess = DecodeSession(inp)
        outs = []
        for t in range(8):
            pr = torch.zeros((2, 4, sess.probs_stride()), device="cuda")
            sess.step(probs=pr)
            torch.cuda.synchronize()
            sums = pr.double().sum(-1)
            assert torch.all((sums - 1).abs() < 1e-5), sums
            outs.append((sess.out.clone(), pr.clone(), sess.cum.clone(), sess.tier.clone()))
        results.append(outs)
    for a, b in zip(*results):
        for x, y in zip(a, b):
            assert torch.equal(x, y)


def test_score_only_matches_decode(gpu_lib):
    import ctypes as C
    from kv_cache_compression_gqa_amd import abi
    inp = synth.make_decode(configs.TINY, steps=1)
    s1, s2 = DecodeSession(inp), DecodeSession(inp)
    s1.step(route=False)
    args = s2.decode_args(0, score_only=True)
    ws = s2.workspace(args)
    sa = abi.KvcWindowScoreArgs(cache=C.pointer(s2._cache), step=C.pointer(args))
    abi.check(abi.lib().kvc_score(abi.KVC_SCORE_WINDOWS, C.byref(sa), abi.ptr(ws), s2._ws_bytes,
                                  abi.stream_handle()), "kvc_score")
    torch.cuda.synchronize()
    assert torch.equal(s1.cum, s2.cum)
    assert torch.equal(s1.tail_len, s2.tail_len)
    assert torch.all(s2.out == 0)


def test_batched_32_layers_batch_16_full_size(gpu_lib):
    """4096 units (32 layers x batch 16 x 8 KV heads), lengths uniform in [4096, 8192] per sequence, 25% FULL +
    25% INT2 per unit, routing after every step: every unit runs on the GPU; sampled units across layers,
    sequences and heads follow the oracle exactly (outputs, probabilities, mass and cum every step; tiers,
    lists, ledger and promoted copies at every routing event). Every layer of a (sequence, KV head) holds its
    windows in an order of its own and takes per-unit step inputs, so four layers of one (sequence, KV head)
    are followed and their outputs must differ: a read or write of another layer's unit cannot pass."""
    cfg = configs.BATCHED_32L_B16
    inp, plan = synth.make_decode_shared_layers(cfg)
    print(f"batched: {cfg.n_units} units, lengths {sorted(set(inp.lengths.tolist()))[:3]}..", flush=True)
    same_bg = [cfg.unit_index(l, 5, 3) for l in (0, 1, 17, 31)]
    check = sorted(set([0, 9, 130, 1234, 2048 + 77, cfg.n_units - 1] + same_bg))
    _, _, out = run_decode_parity(cfg, inp=inp, plan=plan, check_units=check, probs=True)
    for i, a in enumerate(same_bg):
        for b in same_bg[i + 1:]:
            assert not np.allclose(out[a], out[b], rtol=1e-2, atol=0.0), f"units {a} and {b} give the same output"


def test_one_round_launch_a_few_tasks_over(gpu_lib):
    """64 units whose step has 4 tasks more than one round of 8-wave workgroups holds (8 per unit on a 256-CU
    GPU): the launch spills a few workgroups into a second round. Without and with probabilities, against the
    oracle."""
    cfg = dataclasses.replace(configs.LLAMA3_8B_LAYER_32K, name="extra_tasks", layers=8, context=134 * 32 + 40,
                              steps=8, route_every=4)
    inp = synth.make_decode(cfg)
    log(f"case: {cfg.name}, {cfg.n_units} units, probabilities off then on")
    run_decode_parity(cfg, inp=inp, check_units=[0, 21, 63], probs=False, log=log)
    run_decode_parity(cfg, inp=inp, check_units=[0, 63], probs=True, log=log)


def test_routing_on_a_second_stream_matches_serial(gpu_lib):
    """Routing events issued on a second stream (after the step's decode, waited for by the session's next step),
    with other sessions' steps in between, give bit-identical outputs, scores, tiers, lists and slots to the serial
    order: eagerly, and captured in one HIP graph with the stream fork and join (replayed once)."""
    cfg = configs.TINY
    n_sess, steps = 3, cfg.steps

    def state(s):
        return [s.out.clone(), s.cum.clone(), s.tier.clone(), s.res_list.clone(), s.full_slot.clone(),
                s.ledger_slot.clone(), s.k_full.clone(), s.k_codes.clone()]

    def run(mode):
        sessions = [DecodeSession(synth.make_decode(cfg)) for _ in range(n_sess)]
        for s in sessions:
            s.reserve_workspace(steps)
        rs = None if mode == "serial" else torch.cuda.Stream()
        outs = []

        def issue():
            for t in range(steps):
                for s in sessions:
                    s.step(route_stream=rs)
                    if mode != "graph":
                        outs.append(s.out.clone())
            for s in sessions:
                s.wait_route()

        torch.cuda.synchronize()
        if mode == "graph":
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                issue()
            torch.cuda.synchronize()
            g.replay()
        else:
            issue()
        torch.cuda.synchronize()
        return outs, [state(s) for s in sessions]

    serial_outs, serial_state = run("serial")
    eager_outs, eager_state = run("eager")
    assert len(serial_outs) == len(eager_outs) == n_sess * steps
    for a, b in zip(serial_outs, eager_outs):
        assert torch.equal(a, b)
    for mode_state in (eager_state, run("graph")[1]):
        for sa, sb in zip(serial_state, mode_state):
            for x, y in zip(sa, sb):
                assert torch.equal(x, y)
    log("routing on a second stream: eager and captured runs equal the serial run")

"""Drive the HIP decode path and the oracle side by side on the same seeded inputs and compare them.

Tolerances (fp32 accumulation on the GPU against the fp64 oracle):
  * attention output, per (unit, head) row:  max|g - r| <= 2e-3 * max|r|
  * per-key probabilities, window mass, cumulative score:  |g - r| <= 2e-3 * |r| + 1e-12
  * tiers, resident lists, quantise / promote lists: bit-exact when the oracle's router is fed the GPU's fp32
    cumulative scores (teacher forcing: the oracle then continues on those tiers)
  * ledger codes + metadata and promoted full-precision windows: byte-exact;
  * slots (storage is an implementation choice, so the oracle has none): checked against the library's own
    allocation rule, every slot distinct and inside its pool; the bytes above are read through them.
"""
from __future__ import annotations

import numpy as np
import torch

from kv_cache_compression_gqa_amd import layout, synth
from kv_cache_compression_gqa_amd.session import DecodeSession
from oracle.qevict import QEvictUnit
from oracle.select import EVICTED, FULL, INT2

RTOL = 2e-3


def rel_check(name, g, r, rtol=RTOL, atol=1e-12):
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    assert g.shape == r.shape, (name, g.shape, r.shape)
    bad = np.abs(g - r) > rtol * np.abs(r) + atol
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{name}: {bad.sum()} of {bad.size} out of tolerance, first at {tuple(i)}: "
                             f"gpu={g[tuple(i)]!r} oracle={r[tuple(i)]!r}")


def row_check(name, g, r, rtol=RTOL):
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    for h in range(r.shape[0]):
        err = np.abs(g[h] - r[h]).max()
        lim = rtol * np.abs(r[h]).max()
        assert err <= lim, f"{name} head {h}: max err {err} > {lim}"


def make_oracles(inp, units=None, unit_map=None, summaries=False, plan=None):
    """Oracle units keyed by session unit j (held unit unit_map[j] of ``inp``; with a ``synth.SharedLayers``
    plan, held unit plan.unit_map[j] with its windows in the plan's order)."""
    if plan is not None:
        unit_map = plan.unit_map
    umap = np.arange(len(inp.units)) if unit_map is None else np.asarray(unit_map)
    out = {}
    for j in (range(len(umap)) if units is None else units):
        b = int(umap[j])
        nw = int(inp.n_windows[b])
        t0 = int(inp.tail0[b])
        order = np.arange(nw) if plan is None else plan.window_order(inp, j)
        out[j] = QEvictUnit(inp.k_win[b, order], inp.v_win[b, order], inp.k_tail0[b, :t0], inp.v_tail0[b, :t0],
                            inp.cfg.dtype, summaries=summaries)
    return out


def step_inputs(inp, t, j, unit_map=None, plan=None):
    """(q, k_new, v_new) of session unit j at step t."""
    if plan is not None:
        return plan.q[t, j], plan.k_new[t, j], plan.v_new[t, j]
    b = j if unit_map is None else int(unit_map[j])
    return inp.q[t, b], inp.k_new[t, b], inp.v_new[t, b]


def slot_snapshot(sess: DecodeSession):
    """Host copy of the tables the slot check needs, taken just before a routing event."""
    return dict(tier=sess.tier.cpu().numpy(), full_slot=sess.full_slot.cpu().numpy(),
                ledger_slot=sess.ledger_slot.cpu().numpy(), ledgered=sess.ledgered.cpu().numpy(), FS=sess.FS,
                LS=sess.LS, repacked=sess.repacked)


def expected_slots(before, j, tier_after, repack_to=None):
    """The library's slot rule for unit j (include/kvc.h, kvc_route): windows that stay FULL keep their
    full-precision slot, resident windows that have a ledger copy keep their ledger slot; the free slots of each
    pool, ascending, go to the promoted windows (full-precision) and to the windows demoted for the first time
    (ledger) in ascending window order. ``repack_to``: kvc_repack_full ran after the event, so the FULL windows,
    ascending, hold slots 0, 1, ... Returns ({window: full slot}, {window: ledger slot})."""
    tb, fs, ls, led = (before[k][j] for k in ("tier", "full_slot", "ledger_slot", "ledgered"))
    nw = len(tier_after)
    kept = [w for w in range(nw) if tb[w] == FULL and tier_after[w] == FULL]
    free = sorted(set(range(before["FS"])) - {int(fs[w]) for w in kept})
    exp_full = {w: int(fs[w]) for w in kept}
    for k, w in enumerate(w for w in range(nw) if tb[w] == INT2 and tier_after[w] == FULL):
        exp_full[w] = free[k]
    if repack_to is not None:
        exp_full = {w: i for i, w in enumerate(sorted(exp_full))}
    kept_l = [w for w in range(nw) if led[w] and tier_after[w] != EVICTED]
    free_l = sorted(set(range(before["LS"])) - {int(ls[w]) for w in kept_l})
    exp_led = {w: int(ls[w]) for w in kept_l}
    for k, w in enumerate(w for w in range(nw) if tb[w] == FULL and tier_after[w] == INT2 and not led[w]):
        exp_led[w] = free_l[k]
    return exp_full, exp_led


def compare_route(sess: DecodeSession, oracles, gpu_cum, before):
    """Routing of the oracle units (fed the GPU's cumulative scores) against the session: tiers, resident lists,
    plan lists, ledger flags and bytes, full-precision copies of resident FULL windows, and the slots every window
    holds (the library's allocation rule; the copies are read through them). ``before``: slot_snapshot() taken
    just before the event. Only the checked units' rows are copied to the host."""
    keys = sorted(oracles)
    sel = torch.tensor(keys, dtype=torch.int64, device=sess.device)
    g = lambda t: t.index_select(0, sel).cpu().numpy()  # noqa: E731
    tier, res, nf, nq = g(sess.tier), g(sess.res_list), g(sess.n_full), g(sess.n_int2)
    rslot, fslot, lslot = g(sess.res_slot), g(sess.full_slot), g(sess.ledger_slot)
    qn, ql, pn, pl, led = g(sess.n_quant), g(sess.quant_list), g(sess.n_promo), g(sess.promo_list), g(sess.ledgered)
    kc = g(sess.k_codes)
    vc = g(sess.v_codes).view(np.uint16)
    km = g(sess.k_meta).view(np.uint32)
    vm = g(sess.v_meta).view(np.uint32)
    kw = g(sess.k_full).view(np.uint16)
    vw = g(sess.v_full).view(np.uint16)
    repacked_now = sess.repacked and not before["repacked"]
    for r, j in enumerate(keys):
        o = oracles[j]
        nw = o.n_windows
        plan = o.route(int(sess.bf_host[j]), int(sess.bq_host[j]), scores=gpu_cum[j, :nw])
        np.testing.assert_array_equal(tier[r, :nw], o.tier, err_msg=f"tiers unit {j}")
        full, q2 = o.resident_windows()
        assert nf[r] == full.size and nq[r] == q2.size
        np.testing.assert_array_equal(res[r, :nf[r]], full)
        np.testing.assert_array_equal(res[r, nf[r]:nf[r] + nq[r]], q2)
        np.testing.assert_array_equal(ql[r, :qn[r]], plan.quantized)
        np.testing.assert_array_equal(pl[r, :pn[r]], plan.promoted)
        for w in range(nw):
            assert bool(led[r, w]) == (w in o.ledger), f"ledger flag unit {j} window {w}"
        exp_full, exp_led = expected_slots(before, j, o.tier, sess.FS if repacked_now else None)
        assert sorted(exp_full) == full.tolist() and sorted(exp_led) == sorted(o.ledger)
        for w, sl in exp_full.items():
            assert fslot[r, w] == sl, f"full slot unit {j} window {w}: {fslot[r, w]} != {sl}"
        for w, sl in exp_led.items():
            assert lslot[r, w] == sl, f"ledger slot unit {j} window {w}: {lslot[r, w]} != {sl}"
        np.testing.assert_array_equal(rslot[r, :nf[r]], [exp_full[w] for w in full], err_msg=f"res_slot {j}")
        np.testing.assert_array_equal(rslot[r, nf[r]:nf[r] + nq[r]], [exp_led[w] for w in q2], err_msg=f"res_slot {j}")
        assert all(0 <= sl < sess.FS for sl in exp_full.values()) and len(set(exp_full.values())) == len(exp_full)
        assert all(0 <= sl < sess.LS for sl in exp_led.values()) and len(set(exp_led.values())) == len(exp_led)
        for w, e in o.ledger.items():
            sl = exp_led[w]
            assert kc[r, sl].tobytes() == layout.k_codes_to_lib(e["kc"]).tobytes(), f"K codes unit {j} window {w}"
            assert vc[r, sl].tobytes() == layout.v_codes_to_lib(e["vc"]).tobytes(), f"V codes unit {j} window {w}"
            assert km[r, sl].tobytes() == layout.k_meta_to_lib(e["ks"], e["kz"]).tobytes(), f"K meta {j} {w}"
            assert vm[r, sl].tobytes() == layout.v_meta_to_lib(e["vs"], e["vz"]).tobytes(), f"V meta {j} {w}"
        for w in full:
            sl = exp_full[int(w)]
            assert kw[r, sl].tobytes() == o.kw[w].tobytes(), f"K full copy unit {j} window {w}"
            assert layout.v_win_from_lib(vw[r, sl]).tobytes() == o.vw[w].tobytes(), f"V full copy unit {j} window {w}"
    if sess.summaries:
        ns, ks, vs = g(sess.n_sum), g(sess.k_sum).view(np.uint16), g(sess.v_sum).view(np.uint16)
        for r, j in enumerate(keys):
            o = oracles[j]
            assert ns[r] == len(o.sum_k), f"summary count unit {j}: {ns[r]} vs {len(o.sum_k)}"
            vrows = ks.shape[1]
            vsum = vs[r].transpose(0, 2, 1).reshape(vrows, -1)   # [SM/32][D][32] -> [SM][D]
            for i in range(len(o.sum_k)):
                assert ks[r, i].tobytes() == o.sum_k[i].tobytes(), f"K summary {i} unit {j}"
                assert vsum[i].tobytes() == o.sum_v[i].tobytes(), f"V summary {i} unit {j}"


def run_decode_parity(cfg, units=None, steps=None, check_units=None, check_steps=None, probs=True, log=print,
                      inp=None, unit_map=None, score_schedule="every", token_weight=None, oracle_weight=None,
                      summaries=False, plan=None):
    """Run ``steps`` decode steps (routing on the workload's cadence) on the GPU for every unit, and on the oracle
    for the units in ``check_units`` (default all; units are independent, so a sample of them is followed exactly).
    ``score_schedule`` "event" adds the window mass to the cumulative score only at routing-event steps.
    ``token_weight`` (device [U][G][S] float32) weights the window score on the GPU and ``oracle_weight`` (host
    [U][G][S]) on the oracle side.
    Outputs are compared at every step in ``check_steps`` (default all); routing at every event. ``inp`` and
    ``unit_map`` (optional) give held inputs and the held unit each session unit starts from; ``plan`` (a
    ``synth.SharedLayers``) gives it with per-unit window order and per-step inputs. Returns (session, oracles,
    last GPU output [U][G][D])."""
    if inp is None:
        inp = synth.make_decode(cfg, units=units, steps=steps)
    S = inp.q.shape[0]
    sess = DecodeSession(inp, unit_map=unit_map, score_schedule=score_schedule, summaries=summaries, plan=plan)
    U = sess.U
    umap = sess.unit_map
    oracles = make_oracles(inp, check_units, unit_map, summaries=summaries, plan=plan)
    check_steps = set(range(S)) if check_steps is None else set(check_steps)
    for t in range(S):
        stride = sess.probs_stride()
        pr = torch.zeros((U, sess.G, stride), dtype=torch.float32, device=sess.device) if probs else None
        mass = torch.zeros((U, sess.NW), dtype=torch.float32, device=sess.device)
        sess.step(probs=pr, mass=mass, route=False, token_weight=token_weight)
        torch.cuda.synchronize()
        out = sess.out.cpu().numpy()
        pr_h = pr.cpu().numpy() if probs else None
        mass_h = mass.cpu().numpy()
        cum_h = sess.cum.cpu().numpy()
        for j, o in oracles.items():
            acc = score_schedule == "every" or (cfg.route_every > 0 and (t + 1) % cfg.route_every == 0)
            r = o.step(*step_inputs(inp, t, j, umap, plan), accumulate=acc,
                       token_weight=None if oracle_weight is None else oracle_weight[j])
            if t not in check_steps:
                continue
            nw = oracles[j].n_windows
            row_check(f"out step {t} unit {j}", out[j], r.o)
            if probs:
                rel_check(f"probs step {t} unit {j}", pr_h[j, :, :r.p.shape[1]], r.p)
            rel_check(f"mass step {t} unit {j}", mass_h[j, :nw], r.mass)
            rel_check(f"cum step {t} unit {j}", cum_h[j, :nw], oracles[j].cum)
        if cfg.route_every > 0 and (t + 1) % cfg.route_every == 0:
            gpu_cum = sess.cum.cpu().numpy().astype(np.float64)
            before = slot_snapshot(sess)
            sess.route()
            torch.cuda.synchronize()
            compare_route(sess, oracles, gpu_cum, before)
            log(f"step {t + 1}: routed; tiers, lists, ledger and promoted copies match")
    st = sess.device_status()
    assert st == 0, f"device status bits {st:#x}"
    return sess, oracles, out

"""Pins for the oracle's routing diagnostics and the event-only scoring schedule (CPU only): hand-worked counts,
agreement with the oracle router's own transition lists, future missed mass by brute force over the keys of the
full-cache attention and by mass conservation, the perturbation in closed form and exactly zero at full budget,
and the event-only schedule against the every-step one."""
import numpy as np

from kv_cache_compression_gqa_amd import configs, synth
from oracle import attention, diagnostics, qevict
from oracle.fp import storage_to_f64
from oracle.select import EVICTED, FULL, INT2

CFG = configs.TINY
F, Q, E = FULL, INT2, EVICTED


def make_unit(u=0, steps=8):
    inp = synth.make_decode(CFG, units=[u], steps=steps)
    nw = int(inp.n_windows[0])
    t0 = int(inp.tail0[0])
    unit = qevict.QEvictUnit(inp.k_win[0, :nw], inp.v_win[0, :nw], inp.k_tail0[0, :t0], inp.v_tail0[0, :t0],
                             CFG.dtype)
    return inp, unit


def test_route_counts_hand_worked():
    prev = np.array([F, F, Q, Q, E, F], np.int8)
    now = np.array([F, Q, F, E, E, E], np.int8)
    # changed: windows 1, 2, 3, 5; re-entered FULL: window 2; FULL: 0, 2; resident: 0, 1, 2
    assert diagnostics.route_counts(prev, now) == (4, 1, 2, 3)
    assert diagnostics.route_counts(now, now) == (0, 0, 2, 3)
    assert diagnostics.churn(prev, now) == 4 / 6
    # two events: re-entries 1 then 0, FULL windows 2 then 2
    assert diagnostics.global_lir([(prev, now), (now, now)]) == 1 / 4


def test_route_counts_match_router_transition_lists():
    inp, unit = make_unit(steps=16)
    for t in range(16):
        unit.step(inp.q[t, 0], inp.k_new[t, 0], inp.v_new[t, 0])
        if (t + 1) % 4 == 0:
            plan = unit.route(CFG.budget_full, CFG.budget_int2)
            ch, re, nf, nr = diagnostics.route_counts(plan.tier_before, plan.tier_after)
            assert ch == plan.demoted.size + plan.promoted.size + plan.evicted.size
            assert re == plan.promoted.size
            assert nf == min(CFG.budget_full, unit.n_windows)
            assert nr == int(np.count_nonzero(unit.tier != EVICTED))


def test_future_missed_mass_brute_force_and_conservation():
    inp, unit = make_unit(steps=8)
    nw = unit.n_windows
    W = unit.W
    tk, tv = [], []
    for t in range(8):
        unit.step(inp.q[t, 0], inp.k_new[t, 0], inp.v_new[t, 0])
        tk.append(inp.k_new[t, 0])
        tv.append(inp.v_new[t, 0])
        if (t + 1) % 4 == 0:
            unit.route(CFG.budget_full, CFG.budget_int2)
        # full-cache attention at this step (windows in position order, then the tail)
        _, p, _ = qevict.full_cache_attention(inp.k_win[0, :nw], inp.v_win[0, :nw],
                                              np.concatenate([inp.k_tail0[0, :inp.tail0[0]], np.stack(tk)]),
                                              np.concatenate([inp.v_tail0[0, :inp.tail0[0]], np.stack(tv)]),
                                              inp.q[t, 0], CFG.dtype)
        kw = np.concatenate([np.repeat(np.arange(nw), W), np.full(p.shape[1] - nw * W, -1)])
        mass_full = attention.window_mass(p, kw, nw)
        fmm = diagnostics.future_missed_mass(mass_full, unit.tier)
        brute = 0.0
        for i in range(nw * W):   # every key of an evicted window, every head
            if unit.tier[i // W] == EVICTED:
                brute += p[:, i].sum()
        brute /= p.shape[0]
        assert abs(fmm - brute) <= 1e-12
        tail = p[:, nw * W:].sum() / p.shape[0]
        resident = mass_full[unit.tier != EVICTED].sum()
        assert abs(fmm - (1.0 - resident - tail)) <= 1e-12
        if t < 3:
            assert fmm == 0.0   # nothing evicted before the first event


def test_perturbation_closed_form_and_full_budget_zero():
    # two keys with equal logits: o = (v1 + v2) / 2; keeping only the first gives v1; L = sum |v1 - v2| / 2
    rng = np.random.default_rng(5)
    k = rng.standard_normal(128)
    v = rng.standard_normal((2, 128))
    q = rng.standard_normal((1, 128))
    o_full = attention.gqa_decode(q, np.stack([k, k]), v)[2]
    o_kept = attention.gqa_decode(q, k[None], v[:1])[2]
    L = diagnostics.perturbation_l1(o_full, o_kept)
    assert abs(L[0] - np.abs(v[0] - v[1]).sum() / 2) <= 1e-12
    # full budget: the compressed run is the full-cache attention bit for bit, so L is exactly zero
    inp, unit = make_unit(steps=4)
    nw = unit.n_windows
    tk, tv = [], []
    for t in range(4):
        r = unit.step(inp.q[t, 0], inp.k_new[t, 0], inp.v_new[t, 0])
        tk.append(inp.k_new[t, 0])
        tv.append(inp.v_new[t, 0])
        o = qevict.full_cache_attention(inp.k_win[0, :nw], inp.v_win[0, :nw], np.stack(tk), np.stack(tv),
                                        inp.q[t, 0], CFG.dtype)[2]
        assert np.all(diagnostics.perturbation_l1(o, r.o) == 0.0)


def test_event_only_schedule():
    R = 4
    inp, every = make_unit(steps=12)
    _, event = make_unit(steps=12)
    masses = []
    for t in range(12):
        r = every.step(inp.q[t, 0], inp.k_new[t, 0], inp.v_new[t, 0])
        e = event.step(inp.q[t, 0], inp.k_new[t, 0], inp.v_new[t, 0], accumulate=(t + 1) % R == 0)
        masses.append(e.mass)
        if t < R:
            # same tiers so far: same attention; the event schedule holds only the event step's mass
            assert np.array_equal(r.mass, e.mass) and np.array_equal(r.o, e.o)
        if t == R - 1:
            assert np.array_equal(event.cum, e.mass)
            assert np.allclose(every.cum, np.sum(masses, axis=0), rtol=0, atol=1e-15)
        if (t + 1) % R == 0:
            every.route(CFG.budget_full, CFG.budget_int2)
            event.route(CFG.budget_full, CFG.budget_int2)
    # the event schedule's score is the sum of the masses of the event steps only
    assert np.allclose(event.cum, masses[R - 1] + masses[2 * R - 1] + masses[3 * R - 1], rtol=0, atol=1e-15)


def test_weighted_window_mass():
    """The projected-value weighting of the window score: all-ones weights give the plain mass exactly; a weight
    that picks one position gives that key's head-mean probability; constant weights scale the mass; a dense
    random weighting equals the sum written as one matrix product per window."""
    inp, unit = make_unit(steps=6)
    nw, W = unit.n_windows, unit.W
    G = inp.q.shape[2]
    rng = np.random.default_rng(3)
    for t in range(6):
        r = unit.step(inp.q[t, 0], inp.k_new[t, 0], inp.v_new[t, 0])
        kp = unit.key_pos
        ones = np.ones((G, nw * W))
        assert np.array_equal(attention.weighted_window_mass(r.p, kp, ones, nw, W), r.mass)
        assert np.allclose(attention.weighted_window_mass(r.p, kp, 2.5 * ones, nw, W), 2.5 * r.mass, rtol=1e-15)
        pick = np.zeros((G, nw * W))
        j = int(np.flatnonzero(kp >= 0)[5])
        pick[:, kp[j]] = 1.0
        m = attention.weighted_window_mass(r.p, kp, pick, nw, W)
        assert abs(m[kp[j] // W] - r.p[:, j].mean()) <= 1e-15 and np.count_nonzero(m) == 1
        wt = rng.lognormal(size=(G, nw * W))
        m = attention.weighted_window_mass(r.p, kp, wt, nw, W)
        for w in range(nw):
            cols = np.flatnonzero((kp >= 0) & (kp // W == w))
            ref = sum((r.p[:, c] * wt[:, kp[c]]).sum() for c in cols) / G
            assert abs(m[w] - ref) <= 1e-12 * max(1.0, abs(ref))
        if (t + 1) % 3 == 0:
            unit.route(CFG.budget_full, CFG.budget_int2)

"""Drive the HIP decode path and the oracle side by side on the same seeded inputs and compare them.

Tolerances (fp32 accumulation on the GPU against the fp64 oracle):
  * attention output, per (unit, head) row:  max|g - r| <= 2e-3 * max|r|
  * per-key probabilities, window mass, cumulative score:  |g - r| <= 2e-3 * |r| + 1e-12
  * tiers, resident lists, quantise / promote lists: bit-exact when the oracle's router is fed the GPU's fp32
    cumulative scores (teacher forcing: the oracle then continues on those tiers)
  * ledger codes + metadata and promoted full-precision windows: byte-exact.
"""
from __future__ import annotations

import numpy as np
import torch

from kv_cache_compression_gqa_amd import layout, synth
from kv_cache_compression_gqa_amd.session import DecodeSession
from oracle.qevict import QEvictUnit
from oracle.select import FULL, INT2

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


def make_oracles(inp, units=None):
    out = {}
    for j in (range(len(inp.units)) if units is None else units):
        nw = int(inp.n_windows[j])
        t0 = int(inp.tail0[j])
        out[j] = QEvictUnit(inp.k_win[j, :nw], inp.v_win[j, :nw], inp.k_tail0[j, :t0], inp.v_tail0[j, :t0],
                            inp.cfg.dtype)
    return out


def compare_route(sess: DecodeSession, oracles, gpu_cum):
    tier = sess.tier.cpu().numpy()
    res = sess.res_list.cpu().numpy()
    nf = sess.n_full.cpu().numpy()
    nq = sess.n_int2.cpu().numpy()
    qn = sess.n_quant.cpu().numpy()
    ql = sess.quant_list.cpu().numpy()
    pn = sess.n_promo.cpu().numpy()
    pl = sess.promo_list.cpu().numpy()
    led = sess.ledgered.cpu().numpy()
    kc = sess.k_codes.cpu().numpy()
    vc = sess.v_codes.cpu().numpy().view(np.uint16)
    km = sess.k_meta.cpu().numpy().view(np.uint32)
    vm = sess.v_meta.cpu().numpy().view(np.uint32)
    kw = sess.k_win.cpu().numpy().view(np.uint16)
    vw = sess.v_win.cpu().numpy().view(np.uint16)
    for j, o in oracles.items():
        nw = o.n_windows
        plan = o.route(int(sess.bf_host[j]), int(sess.bq_host[j]), scores=gpu_cum[j, :nw])
        np.testing.assert_array_equal(tier[j, :nw], o.tier, err_msg=f"tiers unit {j}")
        full, q2 = o.resident_windows()
        assert nf[j] == full.size and nq[j] == q2.size
        np.testing.assert_array_equal(res[j, :nf[j]], full)
        np.testing.assert_array_equal(res[j, nf[j]:nf[j] + nq[j]], q2)
        np.testing.assert_array_equal(ql[j, :qn[j]], plan.quantized)
        np.testing.assert_array_equal(pl[j, :pn[j]], plan.promoted)
        for w in range(nw):
            assert bool(led[j, w]) == (w in o.ledger), f"ledger flag unit {j} window {w}"
        for w, e in o.ledger.items():
            assert kc[j, w].tobytes() == layout.k_codes_to_lib(e["kc"]).tobytes(), f"K codes unit {j} window {w}"
            assert vc[j, w].tobytes() == layout.v_codes_to_lib(e["vc"]).tobytes(), f"V codes unit {j} window {w}"
            assert km[j, w].tobytes() == layout.k_meta_to_lib(e["ks"], e["kz"]).tobytes(), f"K meta {j} {w}"
            assert vm[j, w].tobytes() == layout.v_meta_to_lib(e["vs"], e["vz"]).tobytes(), f"V meta {j} {w}"
        for w in full:
            assert kw[j, w].tobytes() == o.kw[w].tobytes(), f"K full copy unit {j} window {w}"
            assert layout.v_win_from_lib(vw[j, w]).tobytes() == o.vw[w].tobytes(), f"V full copy unit {j} window {w}"


def run_decode_parity(cfg, units=None, steps=None, check_units=None, check_steps=None, probs=True, log=print):
    """Run ``steps`` decode steps (routing on the workload's cadence) on the GPU for every unit, and on the oracle
    for the units in ``check_units`` (default all; units are independent, so a sample of them is followed exactly).
    Outputs are compared at every step in ``check_steps`` (default all); routing at every event."""
    inp = synth.make_decode(cfg, units=units, steps=steps)
    S = inp.q.shape[0]
    sess = DecodeSession(inp)
    U = len(inp.units)
    oracles = make_oracles(inp, check_units)
    check_steps = set(range(S)) if check_steps is None else set(check_steps)
    for t in range(S):
        stride = sess.probs_stride()
        pr = torch.zeros((U, sess.G, stride), dtype=torch.float32, device=sess.device) if probs else None
        mass = torch.zeros((U, sess.NW), dtype=torch.float32, device=sess.device)
        sess.step(probs=pr, mass=mass, route=False)
        torch.cuda.synchronize()
        out = sess.out.cpu().numpy()
        pr_h = pr.cpu().numpy() if probs else None
        mass_h = mass.cpu().numpy()
        cum_h = sess.cum.cpu().numpy()
        for j, o in oracles.items():
            r = o.step(inp.q[t, j], inp.k_new[t, j], inp.v_new[t, j])
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
            sess.route()
            torch.cuda.synchronize()
            compare_route(sess, oracles, gpu_cum)
            log(f"step {t + 1}: routed; tiers, lists, ledger and promoted copies match")
    st = sess.device_status()
    assert st == 0, f"device status bits {st:#x}"
    return sess, oracles

"""Throughput of the compressed-KV GQA decode step on one MI355X.

Workload: one Llama-3-8B-shaped attention layer at 32K context (batch 1, 32 query heads / 8 KV heads, head_dim
128, bf16 K/V, window 32, 20% of windows full precision + 30% INT2 + 50% evicted, routing every 16 steps).
A step is one decode step of that schedule in its routed steady state: append the new token, attend over the
FULL + INT2 + tail keys with the window mass and cumulative score fused in, and — every 16th step — re-route the
windows (radix select), quantise first demotions into the write-once ledger and promote by dequantisation.

Cold caches: R = 16 independent replicas (distinct seeds) are stepped round-robin; a routed step touches 34.4 MB
per replica, so 15 other replicas' 516 MB pass between two visits to one, twice the 256 MB Infinity Cache.
Warm-up takes every replica through its first 16 full-cache steps and first routing event, then replica r takes
floor(16 r / R) more steps, so the replicas' routing events are spread evenly over the round-robin and a timed
window of K steps holds about K / 16 of them (reported as routing_events_timed). The K timed steps are captured
in one HIP graph and replayed once between barriers.

value  = KV tokens scored + routed + attended per second = sum over timed steps of the resident positions of the
         sequence (FULL and INT2 window tokens + tail + new token) / wall time.
roofline = the decode kernels' algorithmic bytes per launch (resident K/V bytes: 512 B per full-precision token,
         96 B per INT2 token incl. its scale/zero words, 512 B per tail token, plus q) / their average duration,
         measured with HIP events recorded around every decode launch inside the timed graph.
cpu_baseline = the CPU oracle (fp64 numpy, one thread) on a bounded sample of the same routed steps.
hbm_read_probe_gbs = the faster of two read-only kernels over 2 GiB (the read ceiling of this GPU): a grid-stride
         streaming read, and 16 KiB per-wave tasks with every load issued up front (the decode kernel's pattern for a
         full-precision window, many rounds); read_floor_one_launch_us = one launch that only loads the routed
         launch's bytes in that per-wave pattern.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--replicas R] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=128)
    ap.add_argument("--replicas", type=int, default=16)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true", help="launch steps eagerly instead of one captured graph")
    ap.add_argument("--event-schedule", action="store_true",
                    help="32K layer: add the window mass to the scores only at routing-event steps (plain decode "
                         "steps in between)")
    ap.add_argument("--summaries", action="store_true",
                    help="32K layer: evicted windows leave span summaries attended with a ln 32 size correction")
    ap.add_argument("--weighted", action="store_true",
                    help="32K layer: weight the window score by CriticalKV's |V W_O|_1 (norms from kvc_score)")
    ap.add_argument("--serial-routing", action="store_true",
                    help="32K layer: run every routing event on the decode stream (no overlap with other replicas)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="also run one plain device-to-device copy of this many MiB (counter calibration)")
    ap.add_argument("--workload", default="llama3_8b_layer_32k",
                    choices=["llama3_8b_layer_32k", "batched_32l_b16", "criticalkv_64k", "dbtrim_128k",
                             "dbtrim_paged_decode_128k", "qevict_diagnostics_32k", "topk_33m"],
                    help="the decode step (default), the CriticalKV prefill selection or the DBTrimKV global budget")
    return ap.parse_args()


def step_bytes_and_tokens(sess, W=32, D=128):
    """Algorithmic HBM bytes and KV tokens of the next decode step of a session (host-side counts)."""
    nf, nq, tl = int(sess.h_full.max()), int(sess.h_int2.max()), int(sess.h_tail.max())
    U, G = sess.U, sess.G
    tok_full, tok_int2, tok_tail = nf * W, nq * W, tl + 1
    per_unit = tok_full * 2 * D * 2 + tok_int2 * 2 * (D // 4 + (D // 32) * 4) + tok_tail * 2 * D * 2 + G * D * 2
    if sess.token_weight is not None:  # one fp32 weight per (window token, head)
        per_unit += (tok_full + tok_int2) * G * 4
    if sess.summaries:  # one key and one value row per summary
        per_unit += int(sess.h_sum.max()) * 2 * D * 2
    positions = tok_full + tok_int2 + tok_tail
    return U * per_unit, positions


def kernel_source_sha(files=("decode_attn.hip", "kvc_internal.h")):
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, "kv_cache_compression_gqa_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profile(name="decode_attn_llama3_8b_layer_32k", files=("decode_attn.hip", "kvc_internal.h")):
    """HBM bytes per launch from the committed rocprofv3 counter summary profiles/<name>_traffic.json, if it was
    taken on the current kernel source (its hash is stored with it); None otherwise."""
    path = os.path.join(ROOT, "profiles", f"{name}_traffic.json")
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_sha") != kernel_source_sha(files):
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(cfg, min_seconds=10.0, max_steps=160):
    """Time the oracle on routed steps of the same workload: every KV-head unit of one layer is taken through its
    full-cache phase and first routing event (untimed), then routed steps (with a routing event every 16) are
    timed, one step of every unit per round, until ``min_seconds`` of CPU work or ``max_steps`` rounds. The oracle
    steps the units one after another in one Python thread; its numpy BLAS pool is held to one thread while it is
    timed, so that ``cores`` is the parallelism it really uses."""
    sys.path.insert(0, ROOT)
    from kv_cache_compression_gqa_amd import synth
    from oracle.qevict import QEvictUnit
    units = cfg.n_units
    inp = synth.make_decode(cfg, steps=cfg.route_every + max_steps)
    ors = []
    for j in range(units):
        nw = int(inp.n_windows[j])
        o = QEvictUnit(inp.k_win[j, :nw], inp.v_win[j, :nw], inp.k_tail0[j, :0], inp.v_tail0[j, :0], cfg.dtype)
        for t in range(cfg.route_every):
            o.step(inp.q[t, j], inp.k_new[t, j], inp.v_new[t, j])
        o.route(*cfg.budgets(nw))
        ors.append(o)
    tokens = 0.0
    rounds = 0
    with _one_thread():
        t0 = time.perf_counter()
        while rounds < max_steps and (time.perf_counter() - t0) < min_seconds:
            t = cfg.route_every + rounds
            for j, o in enumerate(ors):
                r = o.step(inp.q[t, j], inp.k_new[t, j], inp.v_new[t, j])
                tokens += r.p.shape[1] / cfg.hkv    # one unit carries one KV head of the sequence's tokens
                if (t + 1) % cfg.route_every == 0:
                    o.route(*cfg.budgets(o.n_windows))
            rounds += 1
        elapsed = time.perf_counter() - t0
    return {"value": tokens / elapsed, "unit": "KV tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{rounds} routed decode steps (routing every {cfg.route_every}) of all {units} KV-head units "
                      f"of one 32K layer after an untimed full-cache phase; fp64 numpy oracle, units one after "
                      f"another in one thread (BLAS pool held to 1); {elapsed:.1f} s"}


class _one_thread:
    """Holds numpy's BLAS/OpenMP pools to one thread inside the block (threadpoolctl)."""

    def __enter__(self):
        try:
            from threadpoolctl import threadpool_limits
            self._lim = threadpool_limits(limits=1)
        except Exception:  # noqa: BLE001
            self._lim = None
        return self

    def __exit__(self, *exc):
        if self._lim is not None:
            self._lim.unregister()
        return False


def _copy_probe_gbs(gib=2, reps=5):
    """Context for the roofline: the HBM traffic (bytes read + written) of a plain device-to-device copy of a 2 GiB
    buffer (far above the Infinity Cache) on this GPU, GB/s."""
    import torch
    x = torch.ones(gib << 30, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    y.copy_(x)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        y.copy_(x)
    b.record()
    torch.cuda.synchronize()
    gbs = 2 * x.numel() * reps / (a.elapsed_time(b) * 1e-3) / 1e9
    del x, y
    torch.cuda.empty_cache()
    return gbs


def _read_probes(step_bytes, launches=64, gib=2, reps=5):
    """The library's HBM read probes (kvc_probe.h) on a 2 GiB buffer:
    - ``stream_gbs``: a grid-stride streaming read of the whole buffer, GB/s;
    - ``wave_task_gbs``: the whole buffer as 16 KiB per-wave tasks (kvc_probe_wave_read), GB/s; the faster of
      the two is the read ceiling of this GPU;
    - ``wave_us``: one launch that only loads ``step_bytes`` (rounded to 16 KiB tasks) in the decode kernel's
      per-wave pattern, every launch from a different slice of the buffer, ``launches`` launches captured in one
      HIP graph and timed with one event pair on their stream: the floor of one launch that moves those bytes."""
    import torch
    from kv_cache_compression_gqa_amd import abi
    L = abi.lib()
    buf = torch.ones(gib << 30, dtype=torch.uint8, device="cuda")
    wgs = L.kvc_probe_stream_workgroups(0)
    sink = torch.empty(max(wgs, 1 << 16), dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream()
    sh = abi.stream_handle(st)
    abi.check(L.kvc_probe_stream_read(abi.ptr(buf), buf.numel(), 0, abi.ptr(sink), sh), "kvc_probe_stream_read")
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(st)
    for _ in range(reps):
        abi.check(L.kvc_probe_stream_read(abi.ptr(buf), buf.numel(), 0, abi.ptr(sink), sh), "kvc_probe_stream_read")
    b.record(st)
    torch.cuda.synchronize()
    stream_gbs = buf.numel() * reps / (a.elapsed_time(b) * 1e-3) / 1e9
    abi.check(L.kvc_probe_wave_read(abi.ptr(buf), buf.numel(), abi.ptr(sink), sh), "kvc_probe_wave_read")
    torch.cuda.synchronize()
    a.record(st)
    for _ in range(reps):
        abi.check(L.kvc_probe_wave_read(abi.ptr(buf), buf.numel(), abi.ptr(sink), sh), "kvc_probe_wave_read")
    b.record(st)
    torch.cuda.synchronize()
    wave_task_gbs = buf.numel() * reps / (a.elapsed_time(b) * 1e-3) / 1e9
    task = 16384
    nb = max(task, (int(step_bytes) + task - 1) // task * task)
    slices = buf.numel() // nb
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gs = torch.cuda.current_stream()
        for i in range(launches):
            off = (i * 7 % slices) * nb
            abi.check(L.kvc_probe_wave_read(buf.data_ptr() + off, nb, abi.ptr(sink), abi.stream_handle(gs)),
                      "kvc_probe_wave_read")
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    a.record(st)
    g.replay()
    b.record(st)
    torch.cuda.synchronize()
    wave_us = a.elapsed_time(b) * 1e3 / launches
    del g, buf, sink
    torch.cuda.empty_cache()
    return {"stream_gbs": stream_gbs, "wave_task_gbs": wave_task_gbs, "wave_us": wave_us, "wave_bytes": nb}


def _calibration_copy(mib):
    """One plain device-to-device copy of ``mib`` MiB (the reference kernel for scaling the HBM counters)."""
    import torch
    if mib > 0:
        src = torch.ones(mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst


def _criticalkv_projection(cfg):
    """A seeded output projection W_O [Hq*128][Hq*128] ~ N(0, 1/d_model) and observation queries for the norms."""
    import torch
    from kv_cache_compression_gqa_amd import synth
    rng = synth.unit_rng(cfg.seed, 1 << 26)
    dm = cfg.hq * cfg.head_dim
    w_o = synth.to_storage_bits(rng.standard_normal((dm, dm)).astype(np.float32) / np.sqrt(dm), cfg.dtype)
    q_obs = synth.to_storage_bits(rng.standard_normal((cfg.hq, 32, cfg.head_dim)), cfg.dtype)
    dev = lambda a: torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)  # noqa: E731
    return dev(w_o), dev(q_obs)


def _projected_value_norms(sess, inp, w_o, q_obs):
    """|V_i W_O,h|_1 for every prefill position of every unit (units = the layer's KV heads), from
    kvc_score(CRITICALKV); returns the [U][G][n] weights the decode takes."""
    import torch
    from kv_cache_compression_gqa_amd import abi, criticalkv
    U, NW, W, D, G = sess.U, sess.NW, sess.W, sess.D, sess.G
    n = NW * W
    k = sess.k_full.view(torch.bfloat16).view(U, n, D)   # before the first event: slot = window
    v = torch.from_numpy(np.ascontiguousarray(inp.v_win).reshape(U, n, D).view(np.int16)).cuda().view(torch.bfloat16)
    out = criticalkv.scores(q_obs, k, v, w_o, abi.KVC_BF16)
    torch.cuda.synchronize()
    return out["norm"].view(U, G, n)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (every (batch, layer, KV head) "
              "unit is independent, so units would shard over GPUs with no exchange)", file=sys.stderr)
        sys.exit(2)
    if args.workload == "criticalkv_64k":
        return bench_criticalkv(args)
    if args.workload == "dbtrim_128k":
        return bench_dbtrim(args)
    if args.workload == "batched_32l_b16":
        return bench_batched(args)
    if args.workload == "dbtrim_paged_decode_128k":
        return bench_paged_decode(args)
    if args.workload == "qevict_diagnostics_32k":
        return bench_diagnostics(args)
    if args.workload == "topk_33m":
        return bench_topk(args)
    import torch
    sys.path.insert(0, ROOT)
    from kv_cache_compression_gqa_amd import configs, synth
    from kv_cache_compression_gqa_amd.session import DecodeSession

    cfg = configs.LLAMA3_8B_LAYER_32K
    R = args.replicas
    E = cfg.route_every
    # routing phases staggered: after the full-cache phase replica r takes floor(r * E / R) more steps, so the
    # replicas' routing events are spread evenly over the round-robin and any window of >= E steps times its share
    offsets = [(r * E) // R for r in range(R)]
    n_full = E * R
    extra_rounds = max(0, -(-(args.warmup - n_full - sum(offsets)) // R))
    warm_total = n_full + sum(offsets) + extra_rounds * R
    per_rep = E + max(offsets) + extra_rounds + 2 * args.steps // R + 4
    torch.cuda.set_device(0)
    sessions = []
    if args.weighted:
        w_o, q_obs = _criticalkv_projection(cfg)
    for r in range(R):
        inp = synth.make_decode(dataclasses.replace(cfg, seed=cfg.seed * 1000 + r), steps=per_rep)
        s = DecodeSession(inp, tail_max=per_rep + 1, summaries=args.summaries,
                          score_schedule="event" if args.event_schedule else "every")
        s.reserve_workspace(per_rep)
        if args.weighted:
            s.token_weight = _projected_value_norms(s, inp, w_o, q_obs)
        sessions.append(s)
    torch.cuda.synchronize()
    print(f"replicas ready: {R} x {cfg.name}", file=sys.stderr, flush=True)

    # warm-up: every replica through its full-cache phase and first routing event. Those first route_every steps
    # of every replica (full-cache attention, then the first routing event with its quantisation and promotions)
    # are captured in one HIP graph and timed: the full-cache phase of the schedule
    full_plan = [step_bytes_and_tokens(sessions[i % R]) for i in range(R)]
    full_ms = None
    if not args.eager:
        fgraph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(fgraph):
            for i in range(n_full):
                sessions[i % R].step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        fgraph.replay()
        torch.cuda.synchronize()
        full_ms = (time.perf_counter() - t0) / n_full * 1e3
        del fgraph
        for s in sessions:   # the first event moved the FULL windows into the b_full pool (inside the graph)
            s.release_prefill_pool()
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    else:
        for i in range(n_full):
            sessions[i % R].step()
    for r in range(R):
        for _ in range(offsets[r] + extra_rounds):
            sessions[r].step()
    torch.cuda.synchronize()
    print(f"warm-up done ({warm_total} steps; replica offsets {offsets})", file=sys.stderr, flush=True)
    _calibration_copy(args.copy_mib)

    K = args.steps
    plan = []  # (bytes, positions) per timed step, from the host-side counts at the time the step is issued
    events_timed = [0]

    # a replica's routing event runs on a second stream (default priority), after its decode and before its next
    # step, so that the other replicas' decode steps overlap it (independent units, as the layers of a model are)
    route_stream = None if args.serial_routing else torch.cuda.Stream()

    def issue(i, events=None):
        s = sessions[i % R]
        plan.append(step_bytes_and_tokens(s))
        if E > 0 and (s.t + 1) % E == 0:
            events_timed[0] += 1
        s.step(events=events, route_stream=route_stream)

    def join_routes():
        for s in sessions:
            s.wait_route()

    # timed region: K steps, captured in one HIP graph and replayed once (or launched eagerly with --eager)
    graph = None
    if not args.eager:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(K):
                issue(i)
            join_routes()
        torch.cuda.synchronize()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if graph is not None:
        graph.replay()
    else:
        for i in range(K):
            issue(i)
        join_routes()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    timed_plan = list(plan)
    print(f"timed region: {K} steps in {wall * 1e3:.3f} ms", file=sys.stderr, flush=True)

    # kernel timing: the next K decode launches of the same replicas with routing held back, so that only the
    # decode launches (decode_partial + decode_combine) run, captured in one HIP graph (launched eagerly with
    # --eager, behind a busy GPU so that the host has enqueued them all) between one pair of HIP events on the
    # stream they run on; the average launch is the span over K
    plan.clear()

    def issue_decode(i):
        s = sessions[i % R]
        plan.append(step_bytes_and_tokens(s))
        s.step(route=False)

    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if graph is not None:
        kgraph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(kgraph):
            for i in range(K):
                issue_decode(K + i)
        torch.cuda.synchronize()
        ev0.record()
        kgraph.replay()
        ev1.record()
    else:
        busy = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        for _ in range(60):
            busy.fill_(1.0)
        ev0.record()
        for i in range(K):
            issue_decode(K + i)
        ev1.record()
        del busy
    torch.cuda.synchronize()
    kern_ms = [ev0.elapsed_time(ev1) / K]
    kern_plan = list(plan)
    st = [s.device_status() for s in sessions]
    if any(st):
        print(f"device status bits set: {st}", file=sys.stderr)
        sys.exit(1)
    total_bytes = sum(b for b, _ in timed_plan)
    total_pos = sum(p for _, p in timed_plan)
    avg_kern_s = float(np.mean(kern_ms)) * 1e-3
    avg_bytes = sum(b for b, _ in kern_plan) / K
    achieved = avg_bytes / avg_kern_s / 1e9
    # the counters were taken on the plain step
    traffic = None if (args.weighted or args.summaries or args.event_schedule) else traffic_from_profile()
    rec = {
        "metric": "KV tokens scored+routed+attended/s per decode step; % of HBM roofline",
        "value": total_pos / wall,
        "unit": "KV tokens/s",
        "n_gpus": 1, "steps": K, "warmup": warm_total, "ms_per_step": wall / K * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name, "batch": 1, "q_heads": cfg.hq, "kv_heads": cfg.hkv, "head_dim": 128,
                   "context": cfg.context, "window": cfg.window, "tiers": "20% full / 30% int2 / 50% evicted",
                   "route_every": cfg.route_every, "phase": "routed steady state", "replicas": R,
                   "routing_stream": "serial" if args.serial_routing else "second stream, overlapping other replicas",
                   "routing_events_timed": events_timed[0], "replica_step_offsets": offsets,
                   "window_score": "attention mass x |V W_O|_1 (CriticalKV norms)" if args.weighted else
                   "attention mass",
                   "evicted_windows": "span summaries (mean key/value, logit + ln 32)" if args.summaries else "dropped",
                   "score_schedule": "routing events only" if args.event_schedule else "every step",
                   "launch": "eager" if graph is None else "hip graph",
                   "window_bytes_per_replica": sessions[0].window_bytes(),
                   "uncompressed_window_bytes_per_replica": sessions[0].U * sessions[0].NW * 2 * 32 * 128 * 2,
                   "full_cache_phase_ms_per_step": full_ms,
                   "full_cache_phase_bytes_per_step": full_plan[0][0],
                   "schedule_64_steps_ms_per_step": None if full_ms is None else
                   (cfg.route_every * full_ms + (cfg.steps - cfg.route_every) * wall / K * 1e3) / cfg.steps},
        "hbm_roofline_frac_step": total_bytes / wall / (HBM_PEAK_GBS * 1e9),
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "kvc_decode_attn (decode_partial + decode_combine)",
                     "avg_launch_us": avg_kern_s * 1e6,
                     "algorithmic_bytes_per_launch": avg_bytes},
    }
    rec["hbm_copy_probe_gbs"] = _copy_probe_gbs()
    probe = _read_probes(avg_bytes)
    ceiling = max(probe["stream_gbs"], probe["wave_task_gbs"])
    rec["hbm_read_probe_gbs"] = ceiling
    rec["hbm_read_probes_gbs"] = {"stream": probe["stream_gbs"], "wave_tasks_16k": probe["wave_task_gbs"]}
    rec["roofline"]["frac_of_read_probe"] = achieved / ceiling
    rec["read_floor_one_launch_us"] = probe["wave_us"]
    rec["read_floor_bytes"] = probe["wave_bytes"]
    if not args.no_cpu_baseline and not (args.weighted or args.summaries or args.event_schedule):
        print("timing the CPU oracle sample", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = _one_thread_baseline(cpu_baseline, cfg)
    print(json.dumps(rec), flush=True)


def unit_bytes_and_tokens(sess, W=32, D=128):
    """Per-unit algorithmic bytes and resident positions of the next decode step (ragged units)."""
    nf, nq, tl = sess.h_full.astype(np.int64), sess.h_int2.astype(np.int64), sess.h_tail.astype(np.int64)
    per_unit = nf * W * 2 * D * 2 + nq * W * 2 * (D // 4 + (D // 32) * 4) + (tl + 1) * 2 * D * 2 + sess.G * D * 2
    return int(per_unit.sum()), int(((nf + nq) * W + tl + 1).sum())


def bench_batched(args):
    """Batched multi-layer decode: 32 layers x batch 16 x 8 KV heads (4096 units), lengths uniform in
    [4096, 8192], 25% FULL + 25% INT2 per unit, score + route + quantise/promote + attention every step."""
    import torch
    sys.path.insert(0, ROOT)
    from kv_cache_compression_gqa_amd import configs, synth
    from kv_cache_compression_gqa_amd.session import DecodeSession
    cfg = configs.BATCHED_32L_B16
    K = max(1, min(args.steps, cfg.steps))
    warm = 2
    torch.cuda.set_device(0)
    inp, layers = synth.make_decode_shared_layers(cfg, steps=warm + 2 * K)
    sess = DecodeSession(inp, plan=layers, tail_max=int(inp.tail0.max()) + warm + 2 * K + 1)
    sess.reserve_workspace(warm + 2 * K)
    torch.cuda.synchronize()
    print(f"session ready: {cfg.name}, {sess.U} units", file=sys.stderr, flush=True)
    for _ in range(warm):
        sess.step()
    torch.cuda.synchronize()
    _calibration_copy(args.copy_mib)
    plan = []

    def issue(events=None):
        plan.append(unit_bytes_and_tokens(sess))
        sess.step(events=events)

    graph = None
    if not args.eager:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(K):
                issue()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if graph is not None:
        graph.replay()
    else:
        for _ in range(K):
            issue()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    timed = list(plan)
    plan.clear()
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    busy = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    for _ in range(20):
        busy.fill_(1.0)
    for i in range(K):
        issue(events=events[i])
    torch.cuda.synchronize()
    del busy
    if sess.device_status():
        print("device status bits set", file=sys.stderr)
        sys.exit(1)
    kern_ms = [a.elapsed_time(b) for a, b in events]
    avg_bytes = sum(b for b, _ in plan) / K
    avg_s = float(np.mean(kern_ms)) * 1e-3
    positions = sum(p for _, p in timed) / cfg.hkv  # (sequence, layer, position) tokens
    rec = {
        "metric": "KV tokens scored+routed+attended/s per decode step; % of HBM roofline",
        "value": positions / wall, "unit": "KV tokens/s", "n_gpus": 1, "steps": K, "warmup": warm,
        "ms_per_step": wall / K * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name, "layers": cfg.layers, "batch": cfg.batch, "q_heads": cfg.hq,
                   "kv_heads": cfg.hkv, "head_dim": 128, "context": list(cfg.context_range), "window": cfg.window,
                   "tiers": "25% full / 25% int2 / 50% evicted", "route_every": cfg.route_every,
                   "units": sess.U, "launch": "eager" if graph is None else "hip graph"},
        "hbm_roofline_frac_step": sum(b for b, _ in timed) / wall / (HBM_PEAK_GBS * 1e9),
        "roofline": {"bound": "hbm", "achieved": avg_bytes / avg_s / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": avg_bytes / avg_s / 1e9 / HBM_PEAK_GBS,
                     "traffic": traffic_from_profile("decode_batched_32l_b16"),
                     "kernel": "kvc_decode_attn (decode_partial + decode_combine)", "avg_launch_us": avg_s * 1e6,
                     "algorithmic_bytes_per_launch": avg_bytes},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = _one_thread_baseline(cpu_baseline_batched, cfg)
    print(json.dumps(rec), flush=True)


def cpu_baseline_batched(cfg, min_seconds=10.0, n_units=32):
    """The oracle on a sample of the batched workload's units (seeded draws at the workload's sequence lengths):
    each unit's first decode step over its full cache and routing, then routed steps with routing every step,
    one step of every sampled unit per round, until ``min_seconds`` have passed."""
    sys.path.insert(0, ROOT)
    from kv_cache_compression_gqa_amd import synth
    from oracle.qevict import QEvictUnit
    units = list(range(0, cfg.n_units, max(1, cfg.n_units // n_units)))[:n_units]
    max_rounds = 256
    inp = synth.make_decode(cfg, units=units, steps=1 + max_rounds)
    ors = []
    for j in range(len(units)):
        nw, t0 = int(inp.n_windows[j]), int(inp.tail0[j])
        o = QEvictUnit(inp.k_win[j, :nw], inp.v_win[j, :nw], inp.k_tail0[j, :t0], inp.v_tail0[j, :t0], cfg.dtype)
        o.step(inp.q[0, j], inp.k_new[0, j], inp.v_new[0, j])
        o.route(*cfg.budgets(nw))
        ors.append(o)
    tokens, rounds = 0.0, 0
    t0 = time.perf_counter()
    while rounds < max_rounds and time.perf_counter() - t0 < min_seconds:
        t = 1 + rounds
        for j, o in enumerate(ors):
            r = o.step(inp.q[t, j], inp.k_new[t, j], inp.v_new[t, j])
            tokens += r.p.shape[1] / cfg.hkv
            o.route(*cfg.budgets(o.n_windows))
        rounds += 1
    el = time.perf_counter() - t0
    return {"value": tokens / el, "unit": "KV tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(units)} of {cfg.n_units} units (spread over layers, sequences and heads), {rounds} routed "
                      f"steps each with routing every step after an untimed full-cache step; fp64 numpy oracle; "
                      f"{el:.1f} s"}


def _timed_calls(fn, K, W):
    """Run fn W times untimed, then K times with HIP events around each call on the current stream; returns
    (wall seconds for the K calls, list of per-call event milliseconds)."""
    import torch
    for _ in range(W):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, [a.elapsed_time(b) for a, b in ev]


def bench_criticalkv(args):
    """CriticalKV prefill selection of one layer: scores (observation attention A, |V W_O|_1, group means) and the
    two-stage selection, 65536 keys, 32/8 heads, d_model 4096, bf16."""
    import torch
    sys.path.insert(0, ROOT)
    from kv_cache_compression_gqa_amd import abi, configs, criticalkv, synth
    cfg = configs.CRITICALKV_64K
    torch.cuda.set_device(0)
    inp = synth.make_criticalkv(cfg)
    t = {name: torch.from_numpy(getattr(inp, name).view(np.int16)).cuda().view(torch.bfloat16)
         for name in ("q_obs", "k", "v", "w_o")}
    print(f"inputs ready: {cfg.name}", file=sys.stderr, flush=True)
    holder = {}

    def run():
        out = criticalkv.scores(t["q_obs"], t["k"], t["v"], t["w_o"], abi.KVC_BF16)
        holder["idx"] = criticalkv.two_stage(out["a_group"], out["s2_group"], cfg.budget, cfg.alpha)
        holder["out"] = out

    K = max(1, min(args.steps, 10))
    wall, ms = _timed_calls(run, K, 2)
    n, hq, hkv, D, dm = cfg.n_keys, cfg.hq, cfg.hkv, cfg.head_dim, cfg.d_model
    flops_n = 2.0 * n * D * dm * hq                        # V_g W_O,h for every query head
    flops_a = 2 * 2.0 * n * D * cfg.n_obs * hq             # two passes of q.K^T over the observation rows
    avg_s = float(np.mean(ms)) * 1e-3
    rec = {
        "metric": "KV entries scored+selected/s (CriticalKV prefill selection, one layer)",
        "value": n * hkv * K / wall, "unit": "KV entries/s", "n_gpus": 1, "steps": K, "warmup": 2,
        "ms_per_step": wall / K * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name, "n_keys": n, "q_heads": hq, "kv_heads": hkv, "head_dim": D, "d_model": dm,
                   "n_obs": cfg.n_obs, "budget": cfg.budget, "alpha": cfg.alpha},
        "roofline": {"bound": "mfma", "achieved": (flops_n + flops_a) / avg_s / 1e12, "peak": 2500.0,
                     "unit": "TFLOP/s", "frac": (flops_n + flops_a) / avg_s / 1e12 / 2500.0, "traffic": None,
                     "kernel": "kvc_score(CRITICALKV) + kvc_route(TWO_STAGE) (proj_norm dominates)",
                     "avg_launch_us": avg_s * 1e6, "algorithmic_flops_per_launch": flops_n + flops_a},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = _one_thread_baseline(cpu_baseline_criticalkv, cfg, inp)
    print(json.dumps(rec), flush=True)


def cpu_baseline_criticalkv(cfg, inp):
    """The oracle on KV heads of the same layer (each with its G query heads: A, N and S2 over all keys, then
    the two-stage selection), one head at a time until at least 10 s of CPU work or all heads."""
    from oracle import criticalkv as ock
    from oracle import fp as ofp
    G, D = cfg.group, cfg.head_dim
    heads, el = 0, 0.0
    while heads < cfg.hkv and el < 10.0:
        g = heads
        q = ofp.storage_to_f64(inp.q_obs[g * G:(g + 1) * G], cfg.dtype)
        k = ofp.storage_to_f64(inp.k[g:g + 1], cfg.dtype)
        v = ofp.storage_to_f64(inp.v[g:g + 1], cfg.dtype)
        w = ofp.storage_to_f64(inp.w_o[g * G * D:(g + 1) * G * D], cfg.dtype)
        t0 = time.perf_counter()
        A, N, A_g, S2_g = ock.scores(q, k, v, w, G)
        ock.select(A_g, S2_g, cfg.budget, cfg.alpha)
        el += time.perf_counter() - t0
        heads += 1
    return {"value": heads * cfg.n_keys / el, "unit": "KV entries/s", "cores": 1, "kind": "oracle",
            "sample": f"{heads} of {cfg.hkv} KV heads ({G} query heads each, all {cfg.n_keys} keys, d_model "
                      f"{cfg.d_model}): fp64 numpy oracle scores + two-stage selection; {el:.1f} s"}


def _dbtrim_inputs(cfg):
    """The DBTrimKV workload on the device: beta [rows][T] fp32, the source page table [rows][T/page] int32 and the
    K/V pools [rows*T/page][page][128] bf16 (pool row r = seeded table row synth.pool_row_index(r))."""
    import torch
    from kv_cache_compression_gqa_amd import synth
    L, H, T, page = cfg.layers, cfg.hkv, cfg.n_tokens, cfg.page
    rows = L * H
    beta = torch.from_numpy(synth.make_retention_beta(cfg).reshape(rows, T)).cuda()
    pt = torch.from_numpy(synth.make_page_table(cfg).reshape(rows, T // page).astype(np.int32)).cuda()
    n_src = rows * (T // page)
    pools = [synth.device_pool(n_src, page, cfg.head_dim, sd, cfg.dtype) for sd in (cfg.seed * 7 + 1, cfg.seed * 7 + 2)]
    return beta, pt, pools


def bench_dbtrim(args):
    """DBTrimKV global budget: log-retention scores, global top-M and paged compaction over 32 layers x 8 KV heads
    x 131072 tokens (bf16 K/V pools of 2,097,152 16-token pages)."""
    import torch
    sys.path.insert(0, ROOT)
    from kv_cache_compression_gqa_amd import abi, configs, retention, synth
    cfg = configs.DBTRIM_128K
    torch.cuda.set_device(0)
    L, H, T, page, D = cfg.layers, cfg.hkv, cfg.n_tokens, cfg.page, cfg.head_dim
    rows = L * H
    beta, pt, pools = _dbtrim_inputs(cfg)
    out_pages = cfg.keep // page + rows + 1
    print(f"inputs ready: {cfg.name}", file=sys.stderr, flush=True)
    st = {}
    ws = {}

    def score():
        st["s"] = retention.retention_scores(beta, cfg.t, out=st.get("s"))

    def topm():
        st["tm"] = retention.global_topm(st["s"], cfg.keep, workspace=ws.get("tm"))
        ws["tm"] = st["tm"].ws

    def select():  # the score computed inside the top-M passes (never written)
        st["sel"] = retention.global_topm(None, cfg.keep, beta=beta, t=cfg.t, workspace=ws.get("tm"))
        ws["tm"] = st["sel"].ws

    def compact():
        st["c"] = retention.compact_pages(st["sel"].keep, pt, pools[0], pools[1], out_pages, abi.KVC_BF16)

    K = max(1, min(args.steps, 10))
    score()
    topm()
    select()
    _calibration_copy(args.copy_mib)
    res = {}
    for name, fn in (("score", score), ("topm", topm), ("select", select), ("compact", compact)):
        res[name] = _timed_calls(fn, K, 1)
    torch.cuda.synchronize()
    if int(st["tm"].status.item()) or int(st["sel"].status.item()) or int(st["c"].status.item()):
        print("device status bits set", file=sys.stderr)
        sys.exit(1)
    if not torch.equal(st["tm"].keep, st["sel"].keep):
        print("fused selection differs from score + top-M", file=sys.stderr)
        sys.exit(1)
    kept = int(st["c"].lengths.sum().item())
    wall = res["select"][0] + res["compact"][0]  # the pipeline: fused score + top-M, then compaction
    comp_s = float(np.mean(res["compact"][1])) * 1e-3
    comp_bytes = kept * D * 2 * 2 * 2 + rows * T  # K and V rows read and written, plus the keep mask
    rec = {
        "metric": "KV entries scored+selected+compacted/s (DBTrimKV global budget)",
        "value": cfg.n_entries * K / wall, "unit": "KV entries/s", "n_gpus": 1, "steps": K, "warmup": 1,
        "ms_per_step": wall / K * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name, "layers": L, "kv_heads": H, "n_tokens": T, "page": page,
                   "keep": cfg.keep, "pipeline": "score inside the top-M passes, then compaction",
                   "ms_select_fused": float(np.mean(res["select"][1])),
                   "ms_score": float(np.mean(res["score"][1])), "ms_topm_from_scores": float(np.mean(res["topm"][1])),
                   "ms_compact": comp_s * 1e3},
        "roofline": {"bound": "hbm", "achieved": comp_bytes / comp_s / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": comp_bytes / comp_s / 1e9 / HBM_PEAK_GBS,
                     "traffic": traffic_from_profile("dbtrim_global_128k", ("retention.hip", "kvc_internal.h")),
                     "kernel": "kvc_compact_pages (compact_gather dominates)", "avg_launch_us": comp_s * 1e6,
                     "algorithmic_bytes_per_launch": comp_bytes},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = _one_thread_baseline(cpu_baseline_dbtrim, cfg)
    print(json.dumps(rec), flush=True)


def bench_paged_decode(args):
    """Decode attention over the per-row page lists that the DBTrimKV global budget leaves (32 layers x 8 KV heads,
    10% of 131072 positions kept in all, 16-token pages): the budget is taken on the device (scores, top-M,
    compaction), then one decode step (G = 4 query heads per row) attends over every row's kept tokens."""
    import torch
    sys.path.insert(0, ROOT)
    from kv_cache_compression_gqa_amd import abi, configs, retention, synth
    cfg = configs.DBTRIM_128K
    torch.cuda.set_device(0)
    L, H, T, page, D, G = cfg.layers, cfg.hkv, cfg.n_tokens, cfg.page, cfg.head_dim, 4
    rows = L * H
    beta, pt, pools = _dbtrim_inputs(cfg)
    comp = retention.compact_pages(retention.global_topm(retention.retention_scores(beta, cfg.t), cfg.keep).keep, pt,
                                   pools[0], pools[1], cfg.keep // page + rows + 1, abi.KVC_BF16)
    torch.cuda.synchronize()
    if int(comp.status.item()):
        print("device status bits set by the compaction", file=sys.stderr)
        sys.exit(1)
    del beta, pools
    torch.cuda.empty_cache()
    lengths = comp.lengths
    n_pages = comp.n_pages.to(torch.int64)
    max_pages = int(n_pages.max().item())
    col = torch.arange(max_pages, device="cuda", dtype=torch.int64)
    # row r owns the fresh pages page_offset[r] .. page_offset[r] + n_pages[r] - 1, in order
    pl = torch.where(col[None, :] < n_pages[:, None], comp.page_offset.to(torch.int64)[:, None] + col[None, :],
                     torch.full_like(col[None, :], -7)).to(torch.int32).contiguous()
    q = torch.from_numpy(synth.to_storage_bits(synth.unit_rng(cfg.seed, 1 << 25).standard_normal((rows, G, D)),
                                               "bf16").view(np.int16)).cuda().view(torch.bfloat16)
    kp = comp.k.view(-1, page, D)
    vp = comp.v.view(-1, page, D)
    dec = retention.PagedDecoder(rows, G, page, max_pages, abi.KVC_BF16)
    out = torch.empty((rows, G, D), dtype=torch.float32, device="cuda")
    print(f"inputs ready: {cfg.name} paged decode, {int(lengths.sum().item())} tokens", file=sys.stderr, flush=True)
    _calibration_copy(args.copy_mib)
    K = max(1, args.steps)
    wall, ms = _timed_calls(lambda: dec(q, kp, vp, pl, lengths, out=out), K, max(1, args.warmup))
    torch.cuda.synchronize()
    if int(dec.status.item()) or not bool(torch.isfinite(out).all()):
        print("paged decode: device status bits set or non-finite output", file=sys.stderr)
        sys.exit(1)
    kept = int(lengths.sum().item())
    launch_s = float(np.mean(ms)) * 1e-3
    nbytes = kept * D * 2 * 2 + int(n_pages.sum().item()) * 4 + rows * 4 + rows * G * D * (2 + 4)
    rec = {
        "metric": "KV tokens attended/s (decode over the per-row page lists left by the DBTrimKV global budget)",
        "value": kept * K / wall, "unit": "KV tokens/s", "n_gpus": 1, "steps": K, "warmup": max(1, args.warmup),
        "ms_per_step": wall / K * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name + "_paged_decode", "rows": rows, "q_heads_per_row": G, "head_dim": D,
                   "page": page, "kept_tokens": kept, "max_row_tokens": int(lengths.max().item())},
        "roofline": {"bound": "hbm", "achieved": nbytes / launch_s / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": nbytes / launch_s / 1e9 / HBM_PEAK_GBS,
                     "traffic": traffic_from_profile("dbtrim_paged_decode_128k", ("paged_decode.hip", "kvc_internal.h")),
                     "kernel": "kvc_paged_decode_attn (paged_partial + paged_combine)",
                     "avg_launch_us": launch_s * 1e6, "algorithmic_bytes_per_launch": nbytes},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = _one_thread_baseline(cpu_baseline_paged, cfg, G)
    print(json.dumps(rec), flush=True)


def cpu_baseline_paged(cfg, G, min_seconds=10.0):
    """The oracle's paged decode on whole rows of the same length (the workload's mean kept count per row), row
    after row, until at least ``min_seconds`` have passed."""
    from kv_cache_compression_gqa_amd import synth
    from oracle.fp import storage_to_f64
    from oracle.paged import paged_gqa_decode
    n = cfg.keep // (cfg.layers * cfg.hkv)
    lists = synth.make_large_paged_lists([n] * 256, G, cfg.page, seed=91)
    done, el = 0, 0.0
    t0 = time.perf_counter()
    while el < min_seconds:
        r = done % 256
        pos = np.arange(n)
        ids = lists.page_list[r][pos // cfg.page].astype(np.int64) * cfg.page + pos % cfg.page
        K = storage_to_f64(synth.pool_row_bits(ids, cfg.head_dim, lists.k_seed), "bf16").reshape(n, 1, -1)
        V = storage_to_f64(synth.pool_row_bits(ids, cfg.head_dim, lists.v_seed), "bf16").reshape(n, 1, -1)
        paged_gqa_decode(storage_to_f64(lists.q[r], "bf16"), K, V, pos, n, 1)
        done += 1
        el = time.perf_counter() - t0
    return {"value": done * n / el, "unit": "KV tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} rows of {n} kept tokens (the mean row of the workload), G = {G}: fp64 numpy oracle "
                      f"(page gather + decode attention); {el:.1f} s"}


def bench_diagnostics(args):
    """QEvict's dynamics diagnostics on a synthetic run of the 32K layer: the compressed run next to a full-cache
    run of the same inputs (all windows FULL, never routed). Per step: the future missed mass (full-cache attention
    on evicted windows) and the L1 output perturbation per head; per routing event: churn and re-entries into the
    FULL tier. The kernel (kvc_route_diagnostics) is timed with HIP events on the per-step call."""
    import torch
    sys.path.insert(0, ROOT)
    from kv_cache_compression_gqa_amd import configs, synth
    from kv_cache_compression_gqa_amd.session import DecodeSession, route_diagnostics
    cfg = configs.LLAMA3_8B_LAYER_32K
    torch.cuda.set_device(0)
    inp = synth.make_decode(cfg)
    sess = DecodeSession(inp)
    nw = inp.n_windows.astype(np.int32)
    shadow = DecodeSession(inp, budgets=(nw, np.zeros_like(nw)))
    U, NW, G = sess.U, sess.NW, sess.G
    mf = torch.zeros((U, NW), dtype=torch.float32, device="cuda")
    tier_prev = torch.empty_like(sess.tier)
    per_step, per_event = [], []
    for t in range(cfg.steps):
        sess.step(route=False)
        shadow.step(mass=mf, route=False)
        per_step.append(route_diagnostics(sess.tier, sess.n_windows, G, mass_full=mf, o_full=shadow.out,
                                          o=sess.out)[1])
        if (t + 1) % cfg.route_every == 0:
            tier_prev.copy_(sess.tier)
            sess.route()
            per_event.append(route_diagnostics(sess.tier, sess.n_windows, G, tier_prev=tier_prev)[0])
    torch.cuda.synchronize()
    if sess.device_status() or shadow.device_status():
        print("device status bits set", file=sys.stderr)
        sys.exit(1)
    vals = torch.stack(per_step).cpu().numpy()      # [steps][U][1 + G]
    cnts = torch.stack(per_event).cpu().numpy()     # [events][U][4]
    out_norm = float(torch.abs(shadow.out).sum(dim=2).mean().item())
    # the kernel: K calls (every input given) captured in one HIP graph, timed by one pair of HIP events on the
    # stream they run on
    K = max(1, args.steps)
    counts = torch.empty((U, 4), dtype=torch.int32, device="cuda")
    values = torch.empty((U, 1 + G), dtype=torch.float32, device="cuda")

    def fn():
        route_diagnostics(sess.tier, sess.n_windows, G, tier_prev=tier_prev, mass_full=mf, o_full=shadow.out,
                          o=sess.out, counts=counts, values=values)

    for _ in range(max(1, args.warmup)):
        fn()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(K):
            fn()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    graph.replay()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    call_s = ev0.elapsed_time(ev1) / K * 1e-3
    nbytes = U * NW * (1 + 1 + 4) + 2 * U * G * 128 * 4 + U * 4 + U * (4 * 4 + (1 + G) * 4)
    R = cfg.route_every
    rec = {
        "metric": "KV windows diagnosed/s (QEvict churn, re-entries, future missed mass; CriticalKV L1 perturbation)",
        "value": U * NW * K / wall, "unit": "windows/s", "n_gpus": 1, "steps": K, "warmup": max(1, args.warmup),
        "ms_per_step": wall / K * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": cfg.name + "_diagnostics", "units": U, "windows": NW, "steps": cfg.steps,
                   "route_every": R},
        "diagnostics": {
            "future_missed_mass_mean_routed_steps": float(vals[R:, :, 0].mean()),
            "future_missed_mass_last_step": float(vals[-1, :, 0].mean()),
            "churn_per_event": [float(c) for c in (cnts[:, :, 0].sum(1) / (U * NW))],
            "reentries_per_event": [int(c) for c in cnts[:, :, 1].sum(1)],
            "global_lir": float(cnts[:, :, 1].sum() / max(1, cnts[:, :, 2].sum())),
            "l1_perturbation_mean_routed_steps": float(vals[R:, :, 1:].mean()),
            "full_cache_output_l1_mean": out_norm},
        "roofline": {"bound": "hbm", "achieved": nbytes / call_s / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": nbytes / call_s / 1e9 / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "kvc_route_diagnostics (diag_kernel, graph-timed; latency-bound: 8 workgroups)",
                     "avg_launch_us": call_s * 1e6, "algorithmic_bytes_per_launch": nbytes},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = _one_thread_baseline(cpu_baseline_diagnostics, U, NW, G)
    print(json.dumps(rec), flush=True)


def cpu_baseline_diagnostics(U, NW, G, min_seconds=10.0):
    """The oracle's diagnostics (counts, future missed mass, L1 perturbation) per unit over seeded tiers, masses and
    outputs of the same shape, repeated until ``min_seconds`` have passed."""
    from oracle import diagnostics
    rng = np.random.default_rng(7)
    prev = rng.integers(0, 3, size=(U, NW)).astype(np.int8)
    now = rng.integers(0, 3, size=(U, NW)).astype(np.int8)
    mass = rng.random((U, NW)) / NW
    of, oc = rng.standard_normal((2, U, G, 128))
    calls, el = 0, 0.0
    t0 = time.perf_counter()
    while el < min_seconds:
        for u in range(U):
            diagnostics.route_counts(prev[u], now[u])
            diagnostics.future_missed_mass(mass[u], now[u])
            diagnostics.perturbation_l1(of[u], oc[u])
        calls += 1
        el = time.perf_counter() - t0
    return {"value": calls * U * NW / el, "unit": "windows/s", "cores": 1, "kind": "oracle",
            "sample": f"{calls} calls over {U} units x {NW} windows (seeded tiers, masses, outputs): fp64 numpy "
                      f"oracle; {el:.1f} s"}


def cpu_baseline_dbtrim(cfg, layers=16):
    """The oracle on the first `layers` layers (a budget of 10% of their entries): scores, top-M, compaction plan
    and the row gather of the kept K/V rows."""
    from kv_cache_compression_gqa_amd import synth
    from oracle import dbtrim
    beta = synth.make_retention_beta(cfg, layers=layers)
    pt = synth.make_page_table(cfg, layers=layers)
    m = int(np.floor(cfg.keep_frac * beta.size))
    t0 = time.perf_counter()
    s = dbtrim.log_retention(beta, cfg.t)
    keep = dbtrim.keep_mask(s, m)
    src, lengths, off, n_pages = dbtrim.compact_rows(keep, pt, cfg.page)
    live = src[src >= 0]
    rows_k = synth.pool_row_bits(live, cfg.head_dim, cfg.seed * 7 + 1, cfg.dtype)
    rows_v = synth.pool_row_bits(live, cfg.head_dim, cfg.seed * 7 + 2, cfg.dtype)
    el = time.perf_counter() - t0
    assert rows_k.shape[0] == rows_v.shape[0] == m
    return {"value": beta.size / el, "unit": "KV entries/s", "cores": 1, "kind": "oracle",
            "sample": f"{layers} of {cfg.layers} layers ({beta.size} entries, M = 10%): fp64 numpy oracle scores, "
                      f"top-M, compaction plan and K/V row gather; {el:.1f} s"}


def bench_topk(args):
    """Generic budgeted top-k (kvc_topk) over the DBTrimKV log-retention scores of 32 layers x 8 KV heads x 131072
    tokens (n = 33,554,432 fp32 scores, k = 10% of them), indices written ascending."""
    import ctypes as C

    import torch
    sys.path.insert(0, ROOT)
    from kv_cache_compression_gqa_amd import abi, configs, retention, synth
    cfg = configs.DBTRIM_128K
    torch.cuda.set_device(0)
    rows, T = cfg.layers * cfg.hkv, cfg.n_tokens
    beta = torch.from_numpy(synth.make_retention_beta(cfg).reshape(rows, T)).cuda()
    scores = retention.retention_scores(beta, cfg.t).reshape(-1)
    del beta
    n, k = scores.numel(), cfg.keep
    L = abi.lib()
    need = L.kvc_topk_workspace(n, k)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    idx = torch.empty(k, dtype=torch.int32, device="cuda")
    stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    print(f"inputs ready: topk n={n} k={k}", file=sys.stderr, flush=True)

    def call():
        abi.check(L.kvc_topk(scores.data_ptr(), n, k, idx.data_ptr(), ws.data_ptr(), need, stream), "kvc_topk")

    K = max(1, min(args.steps, 20))
    wall, ms = _timed_calls(call, K, 2)
    got = idx.cpu().numpy()
    if got.size != k or not (np.diff(got) > 0).all():
        print("top-k indices not strictly ascending", file=sys.stderr)
        sys.exit(1)
    call_s = float(np.mean(ms)) * 1e-3
    alg = n * 4 + k * 4  # every score read once, every index written once
    rec = {
        "metric": "scores selected/s (generic budgeted top-k)", "value": n * K / wall, "unit": "scores/s",
        "n_gpus": 1, "steps": K, "warmup": 2, "ms_per_step": wall / K * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "topk_33m", "n": n, "k": k, "scores": "DBTrimKV log-retention, 32 x 8 x 131072"},
        "roofline": {"bound": "hbm", "achieved": alg / call_s / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": alg / call_s / 1e9 / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "kvc_topk (topm passes + count / offsets / write)", "avg_launch_us": call_s * 1e6,
                     "algorithmic_bytes_per_launch": alg},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = _one_thread_baseline(cpu_baseline_topk, cfg)
    print(json.dumps(rec), flush=True)


def cpu_baseline_topk(cfg, layers=32):
    """The oracle's top-k (a full (score desc, index asc) sort) over the retention scores of the first ``layers``
    layers, k = 10%."""
    from kv_cache_compression_gqa_amd import synth
    from oracle import dbtrim, select
    s = dbtrim.log_retention(synth.make_retention_beta(cfg, layers=layers), cfg.t).reshape(-1)
    k = int(np.floor(cfg.keep_frac * s.size))
    t0 = time.perf_counter()
    sel = np.sort(select.topk(s, k))
    el = time.perf_counter() - t0
    assert sel.size == k
    return {"value": s.size / el, "unit": "scores/s", "cores": 1, "kind": "oracle",
            "sample": f"{layers} of {cfg.layers} layers ({s.size} scores, k = 10%): fp64 numpy lexsort; {el:.1f} s"}


def _one_thread_baseline(fn, *args):
    """Runs a CPU baseline with numpy's BLAS/OpenMP pools held to one thread (the oracle's loops are sequential
    Python; its library calls then use one core too), so that its ``cores`` = 1 is the parallelism really used."""
    with _one_thread():
        rec = fn(*args)
    rec["cores"] = 1
    return _with_host(rec)


def _with_host(rec):
    """Adds the host CPU model (first "model name" of /proc/cpuinfo) to a CPU-baseline record."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    rec["cpu_model"] = model
    return rec


if __name__ == "__main__":
    main()

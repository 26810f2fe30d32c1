"""Device-side state of a windowed three-tier decode run and the step/route loop that drives the C ABI.

PyTorch only provides device memory and the stream; every step of the path runs in the HIP library.

A ``DecodeSession`` owns the cache tensors of U units and does, per decode step t (1-based):
    kvc_decode_attn   append (k_t, v_t) to the tail, attend over FULL + INT2 + tail, add the window mass to cum;
    every ``route_every`` steps:
    kvc_route         re-tier the resident windows by cumulative score under the per-unit budgets;
    kvc_quantize_int2 quantise the windows demoted for the first time (write-once ledger);
    kvc_promote       dequantise the windows promoted back to full precision.
The host never reads device state inside a step: the launch bounds it passes (how many FULL / INT2 windows and
tail rows a unit can have) follow from the budgets alone, because routing always fills the tiers in rank order.
"""
from __future__ import annotations

import ctypes as C

import numpy as np
import torch

from . import abi, layout
from .synth import DecodeInputs, SharedLayers


def _dev(a: np.ndarray, dtype, device):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device=device, dtype=dtype)


def _bits(a: np.ndarray, device):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)


class DecodeSession:
    """``unit_map`` (optional, [U] ints): unit u of the session starts from held unit ``unit_map[u]`` of ``inp``
    (its cache, tail and per-step inputs are copied on the device), so that many units can share one seeded
    draw while every unit keeps memory and state of its own. ``plan`` (a ``synth.SharedLayers``, instead of
    ``unit_map``): the same, with every unit's windows rotated as the plan says and per-step inputs of its own."""

    def __init__(self, inp: DecodeInputs, device="cuda", tail_max: int | None = None, steps: int | None = None,
                 budgets=None, unit_map=None, score_schedule: str = "every", summaries: bool = False,
                 plan: SharedLayers | None = None):
        """``score_schedule``: "every" adds every step's window mass to the cumulative score; "event" adds it only
        at the steps that end with a routing event (attention is then materialised for scoring only when the
        routing needs it, and the steps in between are plain decode steps). ``summaries``: every evicted window
        leaves a span summary (mean key and value) that later steps attend with a ln 32 size correction."""
        if score_schedule not in ("every", "event"):
            raise ValueError(score_schedule)
        self.score_schedule = score_schedule
        cfg = inp.cfg
        self.cfg = cfg
        self.inp = inp
        self.device = torch.device(device)
        dev = self.device
        if plan is not None:
            if unit_map is not None:
                raise ValueError("give unit_map or plan, not both")
            unit_map = plan.unit_map
        self.plan = plan
        umap = np.arange(len(inp.units)) if unit_map is None else np.asarray(unit_map, np.int64)
        self.unit_map = umap
        idx = torch.from_numpy(umap).to(dev)

        def expand(t):  # held units -> session units (device gather)
            return t if unit_map is None else t.index_select(0, idx).contiguous()

        def expand_steps(t):
            return t if unit_map is None else t.index_select(1, idx).contiguous()

        def expand_windows(t):  # [U'][NW]... -> [U][NW]...: held unit, windows in the plan's order
            if plan is None:
                return expand(t)
            NWh = t.shape[1]
            nw = torch.from_numpy(inp.n_windows[umap]).to(dev)
            rot = torch.from_numpy(np.asarray(plan.rot, np.int64)).to(dev)
            w = torch.arange(NWh, device=dev, dtype=torch.int64)[None, :]
            src = torch.where(w < nw[:, None], (w + rot[:, None]) % nw.clamp(min=1)[:, None], w)
            flat = (idx[:, None] * NWh + src).reshape(-1)
            return t.reshape(t.shape[0] * NWh, *t.shape[2:]).index_select(0, flat).reshape(len(umap), *t.shape[1:])

        n_windows_u = inp.n_windows[umap]
        tail0_u = inp.tail0[umap]
        U = len(umap)
        NW = inp.n_windows_max
        W, D, G = cfg.window, cfg.head_dim, cfg.group
        S = inp.q.shape[0] if steps is None else steps
        self.U, self.NW, self.G, self.D, self.W = U, NW, G, D, W
        tm = tail_max if tail_max is not None else int(inp.tail0.max()) + S + 1
        self.TM = max(32, (tm + 31) // 32 * 32)
        # budgets
        if budgets is None:
            bf = np.array([cfg.budgets(int(n))[0] for n in n_windows_u], np.int32)
            bq = np.array([cfg.budgets(int(n))[1] for n in n_windows_u], np.int32)
        else:
            bf, bq = (np.asarray(b, np.int32) for b in budgets)
        self.bf_host, self.bq_host = bf, bq
        # slot pools: the prefill pool holds every window (slot = window); the ledger pool one slot per resident
        # window (b_full + b_int2); after the first routing event the FULL windows move into a pool of b_full slots
        # (allocated now, so that no allocation happens inside a routing event) and the prefill pool is released
        self.FS = NW
        self.LS = int(min(NW, max(1, int((bf.astype(np.int64) + bq).max()))))
        self.FS_small = int(min(NW, max(1, int(bf.max()))))
        self.k_full = expand_windows(_bits(inp.k_win, dev))                               # [U][FS][W][D]
        self.v_full = expand_windows(_bits(layout.v_win_to_lib(inp.v_win), dev))          # [U][FS][D][W]
        self._small = (torch.empty((U, self.FS_small, W, D), dtype=torch.int16, device=dev),
                       torch.empty((U, self.FS_small, D, W), dtype=torch.int16, device=dev))
        self._prefill_pool = None   # the prefill pool between the first event and its release
        self.repacked = False
        self._route_done = None     # event of a routing event issued on another stream, not yet waited for
        LS = self.LS
        self.k_codes = torch.zeros((U, LS, W, D // 4), dtype=torch.uint8, device=dev)
        self.v_codes = torch.zeros((U, LS, 16, 4, 8), dtype=torch.int16, device=dev)
        self.k_meta = torch.zeros((U, LS, W, D // 32), dtype=torch.int32, device=dev)
        self.v_meta = torch.zeros((U, LS, 4, 4, 8), dtype=torch.int32, device=dev)
        self.k_tail = torch.zeros((U, self.TM, D), dtype=torch.int16, device=dev)
        self.v_tail = torch.zeros((U, self.TM // W, D, W), dtype=torch.int16, device=dev)
        t0 = int(inp.tail0.max())
        if t0 > 0:
            self.k_tail[:, :t0] = expand(_bits(inp.k_tail0[:, :t0], dev))
            vt = np.zeros((len(inp.units), W, D), np.uint16)
            vt[:, :t0] = inp.v_tail0[:, :t0]
            self.v_tail[:, 0] = expand(_bits(layout.v_tail_to_lib(vt)[:, 0], dev))
        self.tail_len = _dev(tail0_u.astype(np.int32), torch.int32, dev)
        self.n_windows = _dev(n_windows_u.astype(np.int32), torch.int32, dev)
        self.tier = torch.zeros((U, NW), dtype=torch.int8, device=dev)
        self.ledgered = torch.zeros((U, NW), dtype=torch.uint8, device=dev)
        self.cum = torch.zeros((U, NW), dtype=torch.float32, device=dev)
        res = np.tile(np.arange(NW, dtype=np.int32), (U, 1))
        self.res_list = _dev(res, torch.int32, dev)
        self.res_slot = self.res_list.clone()
        self.full_slot = self.res_list.clone()
        self.ledger_slot = torch.full((U, NW), -1, dtype=torch.int32, device=dev)
        self.n_full = _dev(n_windows_u.astype(np.int32), torch.int32, dev)
        self.n_int2 = torch.zeros(U, dtype=torch.int32, device=dev)
        self.status = torch.zeros(1, dtype=torch.int32, device=dev)
        # span summaries of evicted windows (every window is evicted at most once)
        self.summaries = summaries
        self.SM = ((NW + W - 1) // W) * W if summaries else 0
        if summaries:
            self.k_sum = torch.zeros((U, self.SM, D), dtype=torch.int16, device=dev)
            self.v_sum = torch.zeros((U, self.SM // W, D, W), dtype=torch.int16, device=dev)
            self.n_sum = torch.zeros(U, dtype=torch.int32, device=dev)
            self.tier_prev = torch.empty((U, NW), dtype=torch.int8, device=dev)
        else:
            self.k_sum = self.v_sum = self.n_sum = self.tier_prev = None
        self.h_sum = np.zeros(U, np.int64)
        self._sum_ws = None
        # per-step inputs
        if plan is not None:
            self.q = _bits(plan.q, dev)
            self.k_new = _bits(plan.k_new, dev)
            self.v_new = _bits(plan.v_new, dev)
        else:
            self.q = expand_steps(_bits(inp.q, dev))
            self.k_new = expand_steps(_bits(inp.k_new, dev))
            self.v_new = expand_steps(_bits(inp.v_new, dev))
        self.out = torch.zeros((U, G, D), dtype=torch.float32, device=dev)
        self.budget_full = _dev(bf, torch.int32, dev)
        self.budget_int2 = _dev(bq, torch.int32, dev)
        self.quant_list = torch.zeros((U, NW), dtype=torch.int32, device=dev)
        self.promo_list = torch.zeros((U, NW), dtype=torch.int32, device=dev)
        self.n_quant = torch.zeros(U, dtype=torch.int32, device=dev)
        self.n_promo = torch.zeros(U, dtype=torch.int32, device=dev)
        # host-side bounds (never read back from the device)
        self.h_full = n_windows_u.astype(np.int64).copy()
        self.h_int2 = np.zeros(U, np.int64)
        self.h_tail = tail0_u.astype(np.int64).copy()
        self.t = 0
        self._cache = abi.KvcCache(
            n_units=U, group=G, head_dim=D, window=W, n_windows_max=NW, tail_max=self.TM,
            kv_dtype=abi.KVC_BF16 if cfg.dtype == "bf16" else abi.KVC_F16, full_slots=self.FS, ledger_slots=self.LS,
            reserved=0, n_windows=abi.ptr(self.n_windows), k_full=abi.ptr(self.k_full), v_full=abi.ptr(self.v_full),
            k_codes=abi.ptr(self.k_codes), v_codes=abi.ptr(self.v_codes), k_meta=abi.ptr(self.k_meta),
            v_meta=abi.ptr(self.v_meta), k_tail=abi.ptr(self.k_tail), v_tail=abi.ptr(self.v_tail),
            tail_len=abi.ptr(self.tail_len), tier=abi.ptr(self.tier), ledgered=abi.ptr(self.ledgered),
            full_slot=abi.ptr(self.full_slot), ledger_slot=abi.ptr(self.ledger_slot), cum=abi.ptr(self.cum),
            res_list=abi.ptr(self.res_list), res_slot=abi.ptr(self.res_slot), n_full=abi.ptr(self.n_full),
            n_int2=abi.ptr(self.n_int2), status=abi.ptr(self.status), k_sum=abi.ptr(self.k_sum),
            v_sum=abi.ptr(self.v_sum), n_sum=abi.ptr(self.n_sum), sum_max=self.SM, reserved2=0)
        self._ws = None
        self._ws_bytes = 0
        self.token_weight = None  # default per-position weights of the window score (step(token_weight=...))

    # -- bounds -----------------------------------------------------------------------------------------------
    def bounds(self):
        return int(self.h_full.max()), int(self.h_int2.max()), int(self.h_tail.max())

    def probs_stride(self, append=True):
        mf, mq, mt = self.bounds()
        return self.W * (mf + mq) + mt + (1 if append else 0)

    # -- one decode step --------------------------------------------------------------------------------------
    def decode_args(self, t_index: int, out=None, probs=None, mass=None, append=True, accumulate=True,
                    score_only=False, token_weight=None):
        mf, mq, mt = self.bounds()
        a = abi.KvcDecodeArgs(
            q=abi.ptr(self.q[t_index]),
            k_new=abi.ptr(self.k_new[t_index]) if append else None,
            v_new=abi.ptr(self.v_new[t_index]) if append else None,
            out=None if score_only else abi.ptr(self.out if out is None else out),
            probs=abi.ptr(probs), mass=abi.ptr(mass),
            probs_stride=0 if probs is None else int(probs.shape[-1]),
            accumulate_cum=1 if accumulate else 0, max_full=mf, max_int2=mq, max_tail=mt, reserved=0,
            token_weight=abi.ptr(token_weight), weight_stride=0 if token_weight is None else int(token_weight.stride(1)),
            max_summary=int(self.h_sum.max()) if self.summaries else 0, reserved2=0)
        if token_weight is not None:
            assert token_weight.dtype == torch.float32 and token_weight.stride(2) == 1
            assert token_weight.shape[:2] == (self.U, self.G) and token_weight.stride(0) == self.G * token_weight.stride(1)
        return a

    def workspace(self, args: abi.KvcDecodeArgs):
        L = abi.lib()
        need = L.kvc_decode_attn_workspace(C.byref(self._cache), C.byref(args))
        if need == 0:
            raise abi.KvcError(abi.KVC_E_INVALID, "kvc_decode_attn_workspace")
        if self._ws is None or self._ws_bytes < need:
            # any contents will do; sized with headroom so that the tail's growth rarely re-allocates
            self._ws = torch.empty(int(need * 1.25) + 4096, dtype=torch.uint8, device=self.device)
            self._ws_bytes = self._ws.numel()
        return self._ws

    def reserve_workspace(self, extra_steps: int):
        """Allocate the decode workspace for the largest bounds the next ``extra_steps`` steps can reach (so no
        allocation happens later, e.g. while a graph is being captured)."""
        saved = self.h_tail.copy()
        self.h_tail = self.h_tail + extra_steps
        try:
            self.workspace(self.decode_args(0, probs=None))
        finally:
            self.h_tail = saved

    def step(self, probs=None, mass=None, append=True, route=True, stream=None, events=None, token_weight=None,
             static_scratch=False, route_stream=None):
        """Decode step t+1 using the pre-generated inputs of that step; routes when due. ``events`` = (before,
        after) torch events recorded on the stream around the decode launch. ``token_weight`` [U][G][>= NW*W]
        float32 weights every window key's probability per query head in the window score (e.g. the projected-value
        norms of kvc_score(CRITICALKV)); None scores by the plain attention mass. ``static_scratch``: run the step
        through kvc_decode_attn_static (the library's static scratch array; no workspace is allocated).
        ``route_stream``: a due routing event runs there, after this step's decode (event wait), so that other work
        on the step's stream can overlap it; this session's next step waits for it (or call wait_route())."""
        self.wait_route(stream)
        ti = self.t
        R = self.cfg.route_every
        accumulate = self.score_schedule == "every" or (R > 0 and (ti + 1) % R == 0)
        args = self.decode_args(ti, probs=probs, mass=mass, append=append, accumulate=accumulate,
                                token_weight=self.token_weight if token_weight is None else token_weight)
        L = abi.lib()
        if static_scratch:
            if events is not None:
                events[0].record()
            abi.check(L.kvc_decode_attn_static(C.byref(self._cache), C.byref(args), abi.stream_handle(stream)),
                      "kvc_decode_attn_static")
        else:
            ws = self.workspace(args)
            if events is not None:
                events[0].record()
            abi.check(L.kvc_decode_attn(C.byref(self._cache), C.byref(args), abi.ptr(ws), self._ws_bytes,
                                        abi.stream_handle(stream)), "kvc_decode_attn")
        if events is not None:
            events[1].record()
        if append:
            self.h_tail += 1
        self.t += 1
        if route and self.cfg.route_every > 0 and self.t % self.cfg.route_every == 0:
            if route_stream is None:
                self.route(stream=stream)
            else:
                decoded = torch.cuda.Event()
                decoded.record(stream)
                route_stream.wait_event(decoded)
                self.route(stream=route_stream)
                self._route_done = torch.cuda.Event()
                self._route_done.record(route_stream)
        return self.out

    def wait_route(self, stream=None):
        """Makes ``stream`` (default: the current stream) wait for a routing event issued on another stream."""
        if self._route_done is not None:
            (stream if stream is not None else torch.cuda.current_stream()).wait_event(self._route_done)
            self._route_done = None

    # -- routing event ----------------------------------------------------------------------------------------
    def route(self, scores=None, stream=None):
        """One routing event: kvc_route, then (the order the freed slots require) kvc_summarize_evicted,
        kvc_quantize_int2 and kvc_promote; after the first event the FULL windows move into the b_full-slot pool
        (kvc_repack_full), and the prefill pool is released unless a graph is being captured
        (release_prefill_pool() then)."""
        L = abi.lib()
        sh = abi.stream_handle(stream)
        if self.summaries:
            self.tier_prev.copy_(self.tier)
        ra = abi.KvcTierRouteArgs(
            cache=C.pointer(self._cache), scores=abi.ptr(scores), budget_full=abi.ptr(self.budget_full),
            budget_int2=abi.ptr(self.budget_int2), quant_list=abi.ptr(self.quant_list), n_quant=abi.ptr(self.n_quant),
            promo_list=abi.ptr(self.promo_list), n_promo=abi.ptr(self.n_promo))
        abi.check(L.kvc_route(abi.KVC_ROUTE_TIERS, C.byref(ra), None, 0, sh), "kvc_route")
        n_res = self.h_full + self.h_int2
        new_full = np.minimum(self.bf_host, n_res)
        new_int2 = np.minimum(self.bq_host, n_res - new_full)
        evicted = n_res - (new_full + new_int2)
        if self.summaries and int(evicted.max()) > 0:   # reads the slots the event freed: before any rewrite
            if self._sum_ws is None:
                need = L.kvc_summarize_workspace(C.byref(self._cache))
                if need == 0:
                    raise abi.KvcError(abi.KVC_E_INVALID, "kvc_summarize_workspace")
                self._sum_ws = torch.empty(need, dtype=torch.uint8, device=self.device)
            abi.check(L.kvc_summarize_evicted(C.byref(self._cache), abi.ptr(self.tier_prev), int(evicted.max()),
                                              abi.ptr(self._sum_ws), self._sum_ws.numel(), sh),
                      "kvc_summarize_evicted")
            self.h_sum = self.h_sum + evicted
        # bounds of this event's lists: first demotions <= min(b_int2, FULL before); promotions <= min(b_full,
        # INT2 before)
        q_bound = int(np.minimum(self.bq_host, self.h_full).sum())
        p_bound = int(np.minimum(self.bf_host, self.h_int2).sum())
        abi.check(L.kvc_quantize_int2(C.byref(self._cache), abi.ptr(self.quant_list), abi.ptr(self.n_quant),
                                      self.NW, q_bound, sh), "kvc_quantize_int2")
        abi.check(L.kvc_promote(C.byref(self._cache), abi.ptr(self.promo_list), abi.ptr(self.n_promo), self.NW,
                                p_bound, sh), "kvc_promote")
        self.h_full, self.h_int2 = new_full.astype(np.int64), new_int2.astype(np.int64)
        if not self.repacked and self.FS_small < self.FS:
            k_small, v_small = self._small
            abi.check(L.kvc_repack_full(C.byref(self._cache), abi.ptr(k_small), abi.ptr(v_small), self.FS_small, sh),
                      "kvc_repack_full")
            self._prefill_pool = (self.k_full, self.v_full)
            self.k_full, self.v_full = k_small, v_small
            self._cache.k_full, self._cache.v_full = abi.ptr(k_small), abi.ptr(v_small)
            self._cache.full_slots = self.FS = self.FS_small
            self.repacked = True
            if stream is not None:   # the repack reads the prefill pool on that stream
                for t in self._prefill_pool:
                    t.record_stream(stream)
            if not torch.cuda.is_current_stream_capturing():
                self.release_prefill_pool()

    def release_prefill_pool(self):
        """Drop the prefill-sized full-precision pool once the repack that emptied it has been issued (the caching
        allocator reuses the memory only after the stream has passed the repack)."""
        self._prefill_pool = None
        self._small = None

    def window_bytes(self) -> int:
        """Device bytes of window data the session holds: full-precision and ledger pools (prefill pool included
        while it is held)."""
        t = [self.k_full, self.v_full, self.k_codes, self.v_codes, self.k_meta, self.v_meta]
        if self._prefill_pool is not None:
            t += list(self._prefill_pool)
        if self._small is not None and not self.repacked:
            t += list(self._small)
        return int(sum(x.numel() * x.element_size() for x in t))

    def device_status(self, clear=True, stream=None) -> int:
        st = C.c_int32(0)
        abi.check(abi.lib().kvc_read_device_status(C.byref(self._cache), C.byref(st), 1 if clear else 0,
                                                   abi.stream_handle(stream)), "kvc_read_device_status")
        return int(st.value)


def route_diagnostics(tier: torch.Tensor, n_windows: torch.Tensor, group: int, tier_prev=None, mass_full=None,
                      o_full=None, o=None, stream=None, counts=None, values=None):
    """kvc_route_diagnostics: per-unit (changed, entered FULL, FULL, resident) window counts and (future missed
    mass, L1 output perturbation per query head). Returns (counts [U][4] int32, values [U][1 + G] float32) on the
    device (written into ``counts`` / ``values`` when given)."""
    U, NW = tier.shape
    if counts is None:
        counts = torch.empty((U, 4), dtype=torch.int32, device=tier.device)
    if values is None:
        values = torch.empty((U, 1 + group), dtype=torch.float32, device=tier.device)
    assert counts.shape == (U, 4) and values.shape == (U, 1 + group)
    a = abi.KvcDiagArgs(tier_prev=abi.ptr(tier_prev), tier=abi.ptr(tier), n_windows=abi.ptr(n_windows),
                        mass_full=abi.ptr(mass_full), o_full=abi.ptr(o_full), o=abi.ptr(o), counts=abi.ptr(counts),
                        values=abi.ptr(values), n_units=U, n_windows_max=NW, group=group, head_dim=128)
    abi.check(abi.lib().kvc_route_diagnostics(C.byref(a), abi.stream_handle(stream)), "kvc_route_diagnostics")
    return counts, values

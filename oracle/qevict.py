"""QEvict decode run for one unit (batch, layer, KV head), step by step.

Source: QEvict page —
  * "Metodologia: QEvict": the history is split into contiguous windows, routed under a fixed memory budget to
    a full-precision tier, a recoverable INT2 tier that stays attendable, or eviction (lowest-confidence windows
    only, and permanently);
  * "Mecanismos Principais": window importance is attention accumulated over time (cumulative score); demotion
    full -> quantized when importance falls; promotion quantized -> full by dequantisation when the cumulative
    score rises; the write-once ledger quantises a window only at its first demotion and reuses that low-bit copy
    for every later promotion and demotion; attention is materialised to update the scores; GQA is supported.

Readings where the page is silent (each is listed with its reason in the design notes):
  * routing unit = (batch, layer, KV head); per-unit budgets b_full / b_int2 in windows;
  * cumulative score = plain sum over decode steps of the window mass (mean over the G query heads of the
    probability in the window), starting at 0 at the first decode step;
  * order inside a step: append (k_t, v_t) -> attend over the current tiers -> accumulate -> route when
    t % R == 0 (the new tiers serve from step t+1);
  * "materialises attention during routing events" (Implementação) is the alternative schedule: the window mass
    is added to the cumulative score only at the steps that end with a routing event (step(accumulate=False) in
    between); scoring every step is the default;
  * routing ranks the resident windows by (score desc, window asc): ranks [0, b_full) FULL, the next b_int2
    INT2, the rest EVICTED for good;
  * the partial last window and every decode-time token form an unrouted tail that is always attended;
  * a promoted window's full-precision data is RNE_storage(x^) of its ledger copy; its ledger is kept;
  * keys and values of INT2 windows are attended as x^ = fl32(c*s + z);
  * memory follows the tiers ("Metodologia: QEvict": the routing runs under a fixed memory budget): a window holds
    a full-precision copy only while it is FULL (demotion and eviction release it) and a ledger copy from its
    first demotion until its eviction, so after an event at most b_full full-precision copies and at most
    b_full + b_int2 ledger copies exist;
  * with summaries on (SEKV's mixed-resolution term), an evicted window is attended through one summary key and
    value after the tail (oracle.summary), taken from the copy the cache holds for it when it is evicted: its
    full-precision copy if it was FULL, its ledger copy brought back to the storage dtype (RNE_storage(x^), what a
    promotion would store) if it was INT2.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .attention import gqa_decode, weighted_window_mass, window_mass
from .fp import f32_to_storage_rne, storage_to_f64
from .int2 import dequantize, quantize
from .select import EVICTED, FULL, INT2, three_tier
from .summary import SIZE_CORRECTION, summarize


@dataclass
class StepResult:
    logits: np.ndarray      # [G][n_res] (scaled by 1/sqrt(D))
    p: np.ndarray           # [G][n_res]
    o: np.ndarray           # [G][D]
    mass: np.ndarray        # [n_windows] (0 for non-resident windows)
    key_window: np.ndarray  # [n_res] window id of each resident key, -1 for tail keys
    tail_mass: float


@dataclass
class RoutePlan:
    tier_before: np.ndarray
    tier_after: np.ndarray
    quantized: np.ndarray   # windows quantised now (first demotion), ascending
    promoted: np.ndarray    # INT2 -> FULL, ascending
    demoted: np.ndarray     # FULL -> INT2 (all, ascending)
    evicted: np.ndarray     # resident -> EVICTED, ascending


class QEvictUnit:
    def __init__(self, k_win: np.ndarray, v_win: np.ndarray, k_tail: np.ndarray, v_tail: np.ndarray,
                 dtype: str, summaries: bool = False):
        """k_win/v_win [n_w][W][D] storage patterns; k_tail/v_tail [t0][D] storage patterns. ``summaries``: an
        evicted window leaves a summary key and value that are attended with a size correction (SEKV's
        mixed-resolution term; see oracle.summary)."""
        self.summaries = summaries
        self.sum_k, self.sum_v = [], []   # storage patterns [D], in eviction order
        self.dtype = dtype
        k_win = np.asarray(k_win, dtype=np.uint16)
        v_win = np.asarray(v_win, dtype=np.uint16)
        self.n_windows, self.W, self.D = k_win.shape
        # full-precision copies, window -> [W][D] storage patterns: only the windows that are FULL hold one
        self.kw = {w: k_win[w].copy() for w in range(self.n_windows)}
        self.vw = {w: v_win[w].copy() for w in range(self.n_windows)}
        self.tail_k = [np.array(r, np.uint16) for r in k_tail]
        self.tail_v = [np.array(r, np.uint16) for r in v_tail]
        self.tier = np.full(self.n_windows, FULL, np.int8)
        self.cum = np.zeros(self.n_windows, np.float64)
        self.ledger = {}  # w -> dict(kc, ks, kz, vc, vs, vz)
        self.t = 0

    # -- state views ------------------------------------------------------------------------------------------
    def resident_windows(self):
        return np.flatnonzero(self.tier == FULL), np.flatnonzero(self.tier == INT2)

    def copies(self):
        """(full-precision copies, ledger copies) the unit holds."""
        return len(self.kw), len(self.ledger)

    def _ledger_as_storage(self, w: int):
        """Window w's ledger copy brought back to the storage dtype, RNE_storage(x^) (what a promotion stores)."""
        e = self.ledger[w]
        return (f32_to_storage_rne(dequantize(e["kc"], e["ks"], e["kz"]), self.dtype),
                f32_to_storage_rne(dequantize(e["vc"], e["vs"], e["vz"]), self.dtype))

    def window_values(self, w: int):
        """Attended (K, V) of window w in fp64 under its current tier."""
        if self.tier[w] == FULL:
            return storage_to_f64(self.kw[w], self.dtype), storage_to_f64(self.vw[w], self.dtype)
        if self.tier[w] == INT2:
            e = self.ledger[w]
            return (dequantize(e["kc"], e["ks"], e["kz"]).astype(np.float64),
                    dequantize(e["vc"], e["vs"], e["vz"]).astype(np.float64))
        raise ValueError("evicted window has no values")

    def assemble(self):
        """Resident keys in attention order: FULL windows ascending, INT2 windows ascending, then the tail."""
        full, int2 = self.resident_windows()
        Ks, Vs, kw, kp = [], [], [], []
        for w in list(full) + list(int2):
            k, v = self.window_values(int(w))
            Ks.append(k)
            Vs.append(v)
            kw.append(np.full(self.W, w, np.int64))
            kp.append(w * self.W + np.arange(self.W, dtype=np.int64))
        if self.tail_k:
            Ks.append(storage_to_f64(np.stack(self.tail_k), self.dtype))
            Vs.append(storage_to_f64(np.stack(self.tail_v), self.dtype))
            kw.append(np.full(len(self.tail_k), -1, np.int64))
            kp.append(np.full(len(self.tail_k), -1, np.int64))
        if self.sum_k:
            Ks.append(storage_to_f64(np.stack(self.sum_k), self.dtype))
            Vs.append(storage_to_f64(np.stack(self.sum_v), self.dtype))
            kw.append(np.full(len(self.sum_k), -1, np.int64))
            kp.append(np.full(len(self.sum_k), -1, np.int64))
        self.key_pos = np.concatenate(kp)
        n_sum = len(self.sum_k)
        n = sum(len(a) for a in kw)
        self.key_bias = np.concatenate([np.zeros(n - n_sum), np.full(n_sum, SIZE_CORRECTION)])
        return np.concatenate(Ks), np.concatenate(Vs), np.concatenate(kw)

    # -- one decode step -------------------------------------------------------------------------------------
    def step(self, q_bits: np.ndarray, k_new=None, v_new=None, accumulate: bool = True,
             token_weight=None) -> StepResult:
        """One decode step. ``accumulate`` = False leaves the cumulative scores alone (the page's cheaper schedule
        scores only at routing events and decodes plainly in between). ``token_weight`` [G][>= n_windows * W]
        weights each window key's probability per query head (CriticalKV's |V W_O|_1 plugged into the window
        score); None = the plain attention mass."""
        if k_new is not None:
            self.tail_k.append(np.array(k_new, np.uint16))
            self.tail_v.append(np.array(v_new, np.uint16))
        K, V, kw = self.assemble()
        q = storage_to_f64(q_bits, self.dtype)
        s, p, o = gqa_decode(q, K, V, bias=self.key_bias if self.sum_k else None)
        if token_weight is None:
            mass = window_mass(p, kw, self.n_windows)
        else:
            mass = weighted_window_mass(p, self.key_pos, np.asarray(token_weight, np.float64), self.n_windows, self.W)
        if accumulate:
            self.cum += mass
        self.t += 1
        tail_mass = float(p[:, kw < 0].sum() / p.shape[0])
        return StepResult(logits=s, p=p, o=o, mass=mass, key_window=kw, tail_mass=tail_mass)

    # -- routing event ---------------------------------------------------------------------------------------
    def _quantize_window(self, w: int):
        kc, ks, kz = quantize(self.kw[w], self.dtype)
        vc, vs, vz = quantize(self.vw[w], self.dtype)
        self.ledger[w] = dict(kc=kc, ks=ks, kz=kz, vc=vc, vs=vs, vz=vz)

    def route(self, b_full: int, b_int2: int, scores=None) -> RoutePlan:
        """Re-tier the resident windows. ``scores`` replaces the oracle's own cumulative scores (used to feed
        the router the GPU's fp32 scores, so that selections can be compared bit for bit)."""
        sc = self.cum if scores is None else np.asarray(scores, dtype=np.float64)
        before = self.tier.copy()
        after = three_tier(sc, before, b_full, b_int2)
        demoted = np.flatnonzero((before == FULL) & (after == INT2))
        promoted = np.flatnonzero((before == INT2) & (after == FULL))
        evicted = np.flatnonzero((before != EVICTED) & (after == EVICTED))
        quantized = np.array([w for w in demoted if int(w) not in self.ledger], dtype=np.int64)
        for w in quantized:   # first demotion: quantised from the full-precision copy it still holds
            self._quantize_window(int(w))
        for w in evicted:
            w = int(w)
            if self.summaries:   # from the copy the cache holds for the window now
                if before[w] == FULL:
                    ks, vs = self.kw[w], self.vw[w]
                else:
                    ks, vs = self._ledger_as_storage(w)
                self.sum_k.append(summarize(ks, self.dtype))
                self.sum_v.append(summarize(vs, self.dtype))
            self.ledger.pop(w, None)
        for w in list(demoted) + list(evicted):   # their full-precision copies are released
            self.kw.pop(int(w), None)
            self.vw.pop(int(w), None)
        for w in promoted:   # rebuilt from the ledger by dequantisation
            self.kw[int(w)], self.vw[int(w)] = self._ledger_as_storage(int(w))
        self.tier = after
        return RoutePlan(tier_before=before, tier_after=after, quantized=quantized, promoted=promoted,
                         demoted=demoted, evicted=evicted)


def full_cache_attention(k_win: np.ndarray, v_win: np.ndarray, k_tail: np.ndarray, v_tail: np.ndarray,
                         q_bits: np.ndarray, dtype: str):
    """Plain attention over the whole uncompressed cache (windows in position order, then the tail)."""
    D = k_win.shape[-1]
    K = np.concatenate([storage_to_f64(k_win.reshape(-1, D), dtype), storage_to_f64(k_tail.reshape(-1, D), dtype)])
    V = np.concatenate([storage_to_f64(v_win.reshape(-1, D), dtype), storage_to_f64(v_tail.reshape(-1, D), dtype)])
    return gqa_decode(storage_to_f64(q_bits, dtype), K, V)

"""GPU parity of the three-tier routing event (kvc_route, KVC_ROUTE_TIERS) on its tables alone, at every launch shape
the library picks (one wave per unit when units are many, 256 or 1024 threads per unit otherwise), against the
oracle's tiering fed the same fp32 scores and the slot rule of include/kvc.h: tiers, resident lists with their
slots, quantise / promote lists, ledger flags, per-unit counts, and windows past a unit's count left untouched.
Each case runs several events in a row on the state the previous one left (ragged window counts, random starting
tiers and slots, budgets from 0 to past the resident count, scores with many exact ties and signed zeros)."""
import ctypes as C
import sys

import numpy as np
import pytest
import torch

from kv_cache_compression_gqa_amd import abi
from oracle.select import EVICTED, FULL, INT2, three_tier

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


class Tables:
    """Routing tables of U units x NW windows on the device, with the one-byte K/V stand-ins kvc_cache requires
    (the routing event reads none of them)."""

    def __init__(self, U, NW, FS, LS, n_windows, tier, ledgered, full_slot, ledger_slot):
        dev = "cuda"
        i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)  # noqa: E731
        self.U, self.NW, self.FS, self.LS = U, NW, FS, LS
        self.n_windows = i32(n_windows)
        self.tier = torch.from_numpy(np.ascontiguousarray(tier, np.int8)).to(dev)
        self.ledgered = torch.from_numpy(np.ascontiguousarray(ledgered, np.uint8)).to(dev)
        self.full_slot, self.ledger_slot = i32(full_slot), i32(ledger_slot)
        self.cum = torch.zeros((U, NW), dtype=torch.float32, device=dev)
        self.res_list = torch.full((U, NW), -7, dtype=torch.int32, device=dev)
        self.res_slot = torch.full((U, NW), -7, dtype=torch.int32, device=dev)
        self.n_full = torch.zeros(U, dtype=torch.int32, device=dev)
        self.n_int2 = torch.zeros(U, dtype=torch.int32, device=dev)
        self.status = torch.zeros(1, dtype=torch.int32, device=dev)
        self.tail_len = torch.zeros(U, dtype=torch.int32, device=dev)
        self.dummy = torch.zeros(64, dtype=torch.uint8, device=dev)
        d = abi.ptr(self.dummy)
        self.cache = abi.KvcCache(
            n_units=U, group=4, head_dim=128, window=32, n_windows_max=NW, tail_max=32, kv_dtype=abi.KVC_BF16,
            full_slots=FS, ledger_slots=LS, reserved=0, n_windows=abi.ptr(self.n_windows), k_full=d, v_full=d,
            k_codes=d, v_codes=d, k_meta=d, v_meta=d, k_tail=d, v_tail=d, tail_len=abi.ptr(self.tail_len),
            tier=abi.ptr(self.tier), ledgered=abi.ptr(self.ledgered), full_slot=abi.ptr(self.full_slot),
            ledger_slot=abi.ptr(self.ledger_slot), cum=abi.ptr(self.cum), res_list=abi.ptr(self.res_list),
            res_slot=abi.ptr(self.res_slot), n_full=abi.ptr(self.n_full), n_int2=abi.ptr(self.n_int2),
            status=abi.ptr(self.status), k_sum=None, v_sum=None, n_sum=None, sum_max=0, reserved2=0)
        self.quant_list = torch.full((U, NW), -7, dtype=torch.int32, device=dev)
        self.promo_list = torch.full((U, NW), -7, dtype=torch.int32, device=dev)
        self.n_quant = torch.zeros(U, dtype=torch.int32, device=dev)
        self.n_promo = torch.zeros(U, dtype=torch.int32, device=dev)

    def route(self, scores, bf, bq):
        self.budget_full = torch.from_numpy(np.ascontiguousarray(bf, np.int32)).cuda()
        self.budget_int2 = torch.from_numpy(np.ascontiguousarray(bq, np.int32)).cuda()
        self.scores = torch.from_numpy(np.ascontiguousarray(scores, np.float32)).cuda()
        ra = abi.KvcTierRouteArgs(cache=C.pointer(self.cache), scores=abi.ptr(self.scores),
                                  budget_full=abi.ptr(self.budget_full), budget_int2=abi.ptr(self.budget_int2),
                                  quant_list=abi.ptr(self.quant_list), n_quant=abi.ptr(self.n_quant),
                                  promo_list=abi.ptr(self.promo_list), n_promo=abi.ptr(self.n_promo))
        abi.check(abi.lib().kvc_route(abi.KVC_ROUTE_TIERS, C.byref(ra), None, 0, abi.stream_handle()), "kvc_route")
        torch.cuda.synchronize()

    def host(self):
        g = lambda t: t.cpu().numpy()  # noqa: E731
        return {k: g(getattr(self, k)) for k in ("tier", "ledgered", "full_slot", "ledger_slot", "res_list",
                                                 "res_slot", "n_full", "n_int2", "quant_list", "n_quant",
                                                 "promo_list", "n_promo", "status")}


def random_state(rng, U, NW, FS, LS):
    """Per unit: a ragged window count, starting tiers with #FULL <= FS and #ledgered <= LS (every INT2 window
    ledgered, some FULL windows too), distinct slots for the windows that hold one, junk elsewhere."""
    n = rng.integers(0, NW + 1, U)
    n[0], n[-1] = NW, 0
    tier = np.full((U, NW), EVICTED, np.int8)
    led = np.zeros((U, NW), np.uint8)
    fsl = rng.integers(-3, FS + 3, (U, NW)).astype(np.int32)
    lsl = rng.integers(-3, LS + 3, (U, NW)).astype(np.int32)
    for u in range(U):
        w = rng.permutation(int(n[u]))
        nf = min(FS, int(rng.integers(0, n[u] + 1)))
        full = w[:nf]
        rest = w[nf:]
        full_led = full[rng.random(nf) < 0.5]
        room = max(0, LS - full_led.size)
        nq = min(room, int(rng.integers(0, rest.size + 1)))
        int2 = rest[:nq]
        tier[u, full], tier[u, int2] = FULL, INT2
        ledw = np.concatenate([full_led, int2]).astype(np.int64)
        led[u, ledw] = 1
        fsl[u, full] = rng.permutation(FS)[:nf]
        lsl[u, ledw] = rng.permutation(LS)[:ledw.size]
    return n, tier, led, fsl, lsl


def random_scores(rng, U, NW, kind):
    if kind == "ties":
        return np.round(rng.standard_normal((U, NW)), 1).astype(np.float32)
    if kind == "zeros":
        s = rng.choice(np.array([0.0, -0.0, 1.0, -1.0], np.float32), (U, NW))
        return s.astype(np.float32)
    if kind == "const":
        return np.full((U, NW), 0.5, np.float32)
    return (rng.standard_normal((U, NW)) * np.exp(rng.standard_normal((U, NW)) * 4)).astype(np.float32)


def expected(before, n, scores, bf, bq, FS, LS):
    """The event on the host: the oracle's tiers, then the library's slot and list rule (include/kvc.h, kvc_route)."""
    U, NW = before["tier"].shape
    out = {k: before[k].copy() for k in ("tier", "ledgered", "full_slot", "ledger_slot")}
    lists = []
    for u in range(U):
        m = int(n[u])
        tb = before["tier"][u, :m]
        led = before["ledgered"][u, :m]
        ta = three_tier(scores[u, :m].astype(np.float64), tb, max(0, int(bf[u])), max(0, int(bq[u])))
        kept = [w for w in range(m) if tb[w] == FULL and ta[w] == FULL]
        free = sorted(set(range(FS)) - {int(before["full_slot"][u, w]) for w in kept})
        promoted = [w for w in range(m) if tb[w] == INT2 and ta[w] == FULL]
        kept_l = [w for w in range(m) if led[w] and ta[w] != EVICTED]
        free_l = sorted(set(range(LS)) - {int(before["ledger_slot"][u, w]) for w in kept_l})
        quant = [w for w in range(m) if tb[w] == FULL and ta[w] == INT2 and not led[w]]
        for r, w in enumerate(promoted):
            out["full_slot"][u, w] = free[r]
        for r, w in enumerate(quant):
            out["ledger_slot"][u, w] = free_l[r]
        for w in range(m):
            if ta[w] == EVICTED and tb[w] != EVICTED:
                out["ledgered"][u, w] = 0
        out["tier"][u, :m] = ta
        full = [w for w in range(m) if ta[w] == FULL]
        int2 = [w for w in range(m) if ta[w] == INT2]
        slots = [int(out["full_slot"][u, w]) for w in full] + [int(out["ledger_slot"][u, w]) for w in int2]
        lists.append((full, int2, slots, quant, promoted))
    return out, lists


def check_event(got, exp, lists, n, tag):
    assert got["status"][0] == 0, f"{tag}: status {got['status'][0]}"
    for k in ("tier", "ledgered", "full_slot", "ledger_slot"):
        np.testing.assert_array_equal(got[k], exp[k], err_msg=f"{tag}: {k}")
    for u, (full, int2, slots, quant, promoted) in enumerate(lists):
        nf, nq = int(got["n_full"][u]), int(got["n_int2"][u])
        assert (nf, nq) == (len(full), len(int2)), f"{tag}: counts unit {u}"
        np.testing.assert_array_equal(got["res_list"][u, :nf + nq], full + int2, err_msg=f"{tag}: res unit {u}")
        np.testing.assert_array_equal(got["res_slot"][u, :nf + nq], slots, err_msg=f"{tag}: slots unit {u}")
        assert int(got["n_quant"][u]) == len(quant) and int(got["n_promo"][u]) == len(promoted), f"{tag}: {u}"
        np.testing.assert_array_equal(got["quant_list"][u, :len(quant)], quant, err_msg=f"{tag}: quant unit {u}")
        np.testing.assert_array_equal(got["promo_list"][u, :len(promoted)], promoted,
                                      err_msg=f"{tag}: promo unit {u}")


# (units, windows per unit, full slots, ledger slots): 1024 threads per unit (few units; NW up to the 4096
# maximum, 1 to 4 windows per thread), 256 threads (300 units), one wave per unit (1100 units)
SHAPES = [(3, 32, 16, 32), (5, 1000, 300, 700), (2, 4096, 1500, 4096), (4, 1025, 1025, 1025),
          (300, 700, 200, 500), (1100, 250, 80, 200)]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"{s[0]}x{s[1]}" for s in SHAPES])
def test_route_tiers_launch_shapes(gpu_lib, shape):
    U, NW, FS, LS = shape
    rng = np.random.default_rng(U * 7919 + NW)
    n, tier, led, fsl, lsl = random_state(rng, U, NW, FS, LS)
    tb = Tables(U, NW, FS, LS, n, tier, led, fsl, lsl)
    log(f"route shape {shape}")
    for ev, kind in enumerate(("ties", "wide", "zeros", "const")):
        bf = rng.integers(0, FS + 1, U)
        bq = rng.integers(0, LS + 1, U)
        bq = np.minimum(bq, LS - np.minimum(bf, LS))   # the resident windows after the event fit the ledger pool
        bf[0], bq[0] = FS, 0
        if U > 1:
            bf[1], bq[1] = 0, 0
        scores = random_scores(rng, U, NW, kind)
        before = tb.host()
        tb.route(scores, bf, bq)
        got = tb.host()
        exp, lists = expected(before, n, scores, bf, bq, FS, LS)
        check_event(got, exp, lists, n, f"{shape} event {ev} ({kind})")
        # the quantise call that follows a real event marks the first demotions ledgered
        ledg = got["ledgered"].copy()
        for u in range(U):
            ledg[u, got["quant_list"][u, :got["n_quant"][u]]] = 1
        tb.ledgered.copy_(torch.from_numpy(ledg))
    log(f"route shape {shape}: 4 events match")


def test_route_nan_score_on_a_resident_window_is_refused(gpu_lib):
    """A NaN score on a resident window sets KVC_DEV_NAN_SCORE and leaves that unit's tables as they were; NaN on
    an evicted window is ignored."""
    U, NW, FS, LS = 3, 64, 16, 32
    rng = np.random.default_rng(41)
    n, tier, led, fsl, lsl = random_state(rng, U, NW, FS, LS)
    n[:] = NW
    tier[:, :8], led[:, :8] = INT2, 1
    lsl[:, :8] = np.arange(8)
    tier[:, 8:], led[:, 8:] = EVICTED, 0
    tb = Tables(U, NW, FS, LS, n, tier, led, fsl, lsl)
    scores = rng.standard_normal((U, NW)).astype(np.float32)
    scores[0, 3] = np.nan    # resident: unit 0 refused
    scores[1, 20] = np.nan   # evicted: ignored
    before = tb.host()
    tb.route(scores, np.full(U, 4), np.full(U, 2))
    got = tb.host()
    assert got["status"][0] == abi.KVC_DEV_NAN_SCORE
    np.testing.assert_array_equal(got["tier"][0], before["tier"][0])
    for u in (1, 2):
        ta = three_tier(scores[u].astype(np.float64), tier[u], 4, 2)
        np.testing.assert_array_equal(got["tier"][u], ta)


@pytest.mark.parametrize("NW", [64, 700, 4096], ids=["one-wave", "256-threads", "1024-threads"])
def test_route_budgets_up_to_int_max(gpu_lib, NW):
    """Budgets are any int32 >= 0: budget_full + budget_int2 past 2^31 - 1 still ranks every resident window into
    FULL then INT2 (a wrapped sum would drop the INT2 tier)."""
    big = 2**31 - 1
    U = 1100 if NW == 64 else (300 if NW == 700 else 2)
    rng = np.random.default_rng(NW + 5)
    n, tier, led, fsl, lsl = random_state(rng, U, NW, NW, NW)
    tb = Tables(U, NW, NW, NW, n, tier, led, fsl, lsl)
    bf = rng.integers(0, NW + 1, U)
    bf[0] = big
    bq = np.full(U, big)
    bq[1] = rng.integers(0, NW + 1)
    scores = random_scores(rng, U, NW, "ties")
    before = tb.host()
    log(f"route int-max budgets NW={NW}")
    tb.route(scores, bf, bq)
    got = tb.host()
    exp, lists = expected(before, n, scores, bf, bq, NW, NW)
    check_event(got, exp, lists, n, f"int-max budgets NW={NW}")

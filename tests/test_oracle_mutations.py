"""The oracle's pins can fail: each case plants one plausible mistake in an oracle routine (a dropped factor, a wrong
sign, an index off by one, a transposed operand, a flipped tie rule), runs the pins that cover that routine, and
requires at least one of them to fail. The mistakes are planted on the CPU only, through monkeypatch, so the oracle
itself is untouched once each case ends."""
import math

import numpy as np
import pytest

from oracle import attention, criticalkv, dbtrim, diagnostics, fp, int2, paged, qevict, select, summary
from oracle.fp import f16_round_down, f16_round_up, storage_to_f32
from tests import test_oracle_attention_select as pins_as
from tests import test_oracle_criticalkv_dbtrim as pins_cd
from tests import test_oracle_diagnostics as pins_dg
from tests import test_oracle_fp_int2 as pins_int2
from tests import test_oracle_paged as pins_pg
from tests import test_oracle_qevict as pins_qe
from tests import test_oracle_summary as pins_sm

try:
    from exceptiongroup import BaseExceptionGroup  # hypothesis reports several distinct failures as a group
except ImportError:  # pragma: no cover
    BaseExceptionGroup = ()


# what a pin run ends with when it catches a mistake: a failed assertion, or the oracle itself rejecting the
# inconsistent state the mistake leads to (a shape that no longer fits, an index out of range); a TypeError would
# mean a broken case, so it is not counted
CAUGHT = (AssertionError, ValueError, IndexError)


def _fails(pin, *args):
    """True when the pin fails (directly or as a group of failures)."""
    try:
        pin(*args)
    except CAUGHT:
        return True
    except BaseExceptionGroup as eg:  # type: ignore[misc]
        return all(isinstance(e, CAUGHT) for e in eg.exceptions)
    return False


# ---- mutants --------------------------------------------------------------------------------------------------------

def attention_no_scale(q, K, V, bias=None):  # the 1/sqrt(D) dropped
    q, K, V = (np.asarray(a, dtype=np.float64) for a in (q, K, V))
    s = q @ K.T
    e = np.exp(s - s.max(axis=1, keepdims=True))
    p = e / e.sum(axis=1, keepdims=True)
    return s, p, p @ V


def attention_softmax_over_heads(q, K, V, bias=None):  # normalised over the wrong axis
    q, K, V = (np.asarray(a, dtype=np.float64) for a in (q, K, V))
    s = (q @ K.T) / math.sqrt(q.shape[-1])
    e = np.exp(s - s.max())
    p = e / e.sum(axis=0, keepdims=True)
    return s, p, p @ V


def window_mass_no_mean(p, key_window, n_windows):  # the 1/G of the group mean dropped
    mass = np.zeros(n_windows, np.float64)
    sel = key_window >= 0
    np.add.at(mass, key_window[sel], p.sum(axis=0)[sel])
    return mass


def rank_order_ties_high_index_first(scores):  # ties broken by index descending
    sc = np.asarray(scores, dtype=np.float64)
    if np.isnan(sc).any():
        raise ValueError("NaN score")
    return np.lexsort((-np.arange(sc.size), -sc))


def three_tier_budgets_swapped(scores, tier, b_full, b_int2):  # the two budgets exchanged
    return ORIG["three_tier"](scores, tier, b_int2, b_full)


def three_tier_evicted_ranked_again(scores, tier, b_full, b_int2):  # eviction not permanent
    return ORIG["three_tier"](scores, np.zeros_like(np.asarray(tier)), b_full, b_int2)


def two_stage_rounded_share(a, s2, budget, alpha):  # round(alpha * b) instead of floor
    b1 = int(round(alpha * budget + 1e-9)) if alpha * budget % 1 == 0.5 else int(round(alpha * budget))
    i1 = select.topk(a, b1)
    taken = np.zeros(np.asarray(a).size, bool)
    taken[i1] = True
    order2 = select.rank_order(s2)
    return np.sort(np.concatenate([i1, order2[~taken[order2]][:budget - b1]]))


def two_stage_stage1_not_excluded(a, s2, budget, alpha):  # stage 2 may pick stage 1's entries again
    b1 = int(math.floor(alpha * budget))
    i1 = select.topk(a, b1)
    i2 = select.rank_order(s2)[:budget - b1]
    return np.sort(np.concatenate([i1, i2]))


def quantize_thresholds_at_grid(bits, dtype):  # codes by floor((x - z) / s) instead of rounding
    x = storage_to_f32(bits, dtype)
    D = x.shape[-1]
    g = x.reshape(x.shape[:-1] + (D // int2.GROUP, int2.GROUP))
    lo, hi = g.min(axis=-1), g.max(axis=-1)
    z16 = f16_round_down(lo)
    z = z16.astype(np.float32)
    t = ((hi - z).astype(np.float32) / np.float32(3.0)).astype(np.float32)
    flat = hi == z
    s16 = np.where(flat, np.float16(0.0), f16_round_up(np.where(flat, np.float32(1.0), t))).astype(np.float16)
    s = s16.astype(np.float32)
    diff = (g - z[..., None]).astype(np.float32)
    codes = np.zeros(g.shape, np.uint8)
    for k in range(3):
        codes += (diff >= (np.float32(k + 1) * s)[..., None]).astype(np.uint8)
    codes = np.where((s == 0)[..., None], np.uint8(0), codes).astype(np.uint8)
    return codes.reshape(x.shape), s16, z16


def dequantize_zero_subtracted(codes, s16, z16):  # c*s - z
    D = codes.shape[-1]
    c = codes.reshape(codes.shape[:-1] + (D // int2.GROUP, int2.GROUP)).astype(np.float64)
    exact = c * s16.astype(np.float64)[..., None] - z16.astype(np.float64)[..., None]
    return exact.astype(np.float32).reshape(codes.shape)


def log_retention_age_off_by_one(beta, t):  # (t - i - 1) ln beta
    T = beta.shape[-1]
    return (t - 1 - np.arange(T)).astype(np.float64) * np.log(beta.astype(np.float64))


def compact_plan_inclusive_offsets(keep, page):  # page offsets by an inclusive prefix sum
    lengths, _, n_pages, positions = ORIG["compact_plan"](keep, page)
    return lengths, np.cumsum(n_pages).astype(np.int64), n_pages, positions


def projected_norm_l2(v_g, w_o_h):  # an L2 norm in place of L1
    return np.sqrt(((v_g @ w_o_h) ** 2).sum(axis=1))


def observation_mask_off_by_one(q_obs, k, group):  # a query does not see its own position
    Hq, T, D = q_obs.shape
    n = k.shape[1]
    A = np.zeros((Hq, n), np.float64)
    pos = n - T + np.arange(T)
    allowed = np.arange(n)[None, :] < pos[:, None]
    allowed[0, 0] = True
    for h in range(Hq):
        s = (q_obs[h] @ k[h // group].T) / math.sqrt(D)
        s = np.where(allowed, s, -np.inf)
        e = np.where(allowed, np.exp(s - s.max(axis=1, keepdims=True)), 0.0)
        A[h] = (e / e.sum(axis=1, keepdims=True)).sum(axis=0) / T
    return A


def group_score_product_of_means(q_obs, k, v, w_o, group, rows=None):  # mean(A) * mean(N) in place of mean(A N)
    A, N, A_g, _ = ORIG["scores"](q_obs, k, v, w_o, group, rows)
    Hkv = A_g.shape[0]
    S2 = np.stack([A_g[g] * N[g * group:(g + 1) * group].mean(axis=0) for g in range(Hkv)])
    return A, N, A_g, S2


def promoted_copy_truncated(self, w):  # the promoted copy rounded toward zero instead of to nearest
    e = self.ledger[w]
    out = []
    for c, s, z in ((e["kc"], e["ks"], e["kz"]), (e["vc"], e["vs"], e["vz"])):
        x = int2.dequantize(c, s, z)
        if self.dtype == "bf16":
            out.append((x.view(np.uint32) >> 16).astype(np.uint16))
        else:
            t = x.astype(np.float16)
            over = np.abs(t.astype(np.float32)) > np.abs(x)
            t = np.where(over, np.nextafter(t, np.float16(0)), t)
            out.append(t.view(np.uint16))
    return out[0], out[1]


def gather_row_shifted(pool, page_list, length, page):  # row (i + 1) % page of the page: one row late
    rows = [pool[int(page_list[i // page]), (i + 1) % page] for i in range(length)]
    return np.array(rows, dtype=pool.dtype).reshape(length, pool.shape[-1])


def summarize_over_31(rows_bits, dtype):  # the sum divided by one less than the window's length
    x = fp.storage_to_f64(rows_bits, dtype)
    return fp.f32_to_storage_rne((x.sum(axis=0) / (x.shape[0] - 1)).astype(np.float32), dtype)


def missed_mass_counts_int2(mass_full, tier):  # the INT2 windows' mass counted as missed too
    return float(np.asarray(mass_full, np.float64)[np.asarray(tier) != select.FULL].sum())


def perturbation_l2(o_full, o):  # an L2 distance in place of L1
    return np.sqrt(((np.asarray(o_full, np.float64) - np.asarray(o, np.float64)) ** 2).sum(axis=1))


def weighted_mass_head0_weight(p, key_pos, weight, n_windows, window):  # head 0's weights for every head
    return ORIG["weighted_window_mass"](p, key_pos, np.broadcast_to(weight[:1], weight.shape), n_windows, window)


def pack_codes_reversed(codes):  # element 4b + j in bits 6 - 2j .. 7 - 2j
    c = codes.reshape(codes.shape[:-1] + (codes.shape[-1] // 4, 4)).astype(np.uint8)
    out = np.zeros(c.shape[:-1], np.uint8)
    for j in range(4):
        out |= (c[..., j] & 3) << (6 - 2 * j)
    return out


def f16_round_down_by_nearest(x):  # round to nearest in place of toward -inf
    return np.asarray(x, np.float32).astype(np.float16)


ORIG = {"three_tier": select.three_tier, "compact_plan": dbtrim.compact_plan, "scores": criticalkv.scores,
        "weighted_window_mass": attention.weighted_window_mass}

# (case, [(module, attribute, replacement)], [(pin, args)])
CASES = [
    ("attention: 1/sqrt(D) dropped", [(attention, "gqa_decode", attention_no_scale)],
     [(pins_as.test_attention_matches_loops, ())]),
    ("attention: softmax over the heads", [(attention, "gqa_decode", attention_softmax_over_heads)],
     [(pins_as.test_attention_matches_loops, ())]),
    ("window mass: 1/G dropped", [(attention, "window_mass", window_mass_no_mean)],
     [(pins_as.test_window_mass_brute_force_and_conservation, ())]),
    ("ranking: ties to the higher index", [(select, "rank_order", rank_order_ties_high_index_first)],
     [(pins_as.test_topk_matches_sorted, ()), (pins_as.test_global_topm_matches_sorted, ())]),
    ("three tiers: budgets exchanged", [(select, "three_tier", three_tier_budgets_swapped)],
     [(pins_as.test_three_tier_caps_and_permanence, ()),
      (pins_as.test_three_tier_strictly_decreasing_is_a_prefix_split, ())]),
    ("three tiers: evicted windows ranked again", [(select, "three_tier", three_tier_evicted_ranked_again)],
     [(pins_as.test_three_tier_caps_and_permanence, ())]),
    ("two stages: share rounded", [(select, "two_stage", two_stage_rounded_share)],
     [(pins_as.test_two_stage_matches_brute_force, ())]),
    ("two stages: stage-1 picks not excluded", [(select, "two_stage", two_stage_stage1_not_excluded)],
     [(pins_as.test_two_stage_matches_brute_force, ())]),
    ("INT2: codes by floor", [(int2, "quantize", quantize_thresholds_at_grid)],
     [(pins_int2.test_int2_quantiser_normal_rows, ("bf16",)), (pins_int2.test_int2_exact_grid_round_trips, ())]),
    ("INT2: zero subtracted", [(int2, "dequantize", dequantize_zero_subtracted)],
     [(pins_int2.test_int2_exact_grid_round_trips, ())]),
    ("retention: age off by one", [(dbtrim, "log_retention", log_retention_age_off_by_one)],
     [(pins_cd.test_log_retention_order_equals_exact_power_order, ())]),
    ("compaction: inclusive page offsets", [(dbtrim, "compact_plan", compact_plan_inclusive_offsets)],
     [(pins_cd.test_compaction_plan_by_brute_force, ())]),
    ("CriticalKV: L2 norm", [(criticalkv, "projected_value_l1", projected_norm_l2)],
     [(pins_cd.test_projected_norm_by_loops_and_identity, ())]),
    ("CriticalKV: causal mask off by one", [(criticalkv, "observation_attention", observation_mask_off_by_one)],
     [(pins_cd.test_observation_attention_causal_mask_by_loops, ())]),
    ("CriticalKV: product of group means", [(criticalkv, "scores", group_score_product_of_means)],
     [(pins_cd.test_criticalkv_scores_group_means, ())]),
    ("QEvict: promoted copy truncated", [(qevict.QEvictUnit, "_ledger_as_storage", promoted_copy_truncated)],
     [(pins_qe.test_ledger_is_write_once_across_promote_demote_cycles, ())]),
    ("paged: row of the page one late", [(paged, "gather_row", gather_row_shifted)],
     [(pins_pg.test_paged_equals_attention_over_the_contiguous_sequence, ())]),
    ("summary: mean over 31", [(summary, "summarize", summarize_over_31)],
     [(pins_sm.test_summary_is_the_rounded_exact_mean, ())]),
    ("summary: ln 16 size correction", [(summary, "SIZE_CORRECTION", math.log(16.0))],
     [(pins_sm.test_size_correction_matches_identical_tokens, ())]),
    ("diagnostics: INT2 mass counted as missed", [(diagnostics, "future_missed_mass", missed_mass_counts_int2)],
     [(pins_dg.test_future_missed_mass_brute_force_and_conservation, ())]),
    ("diagnostics: L2 perturbation", [(diagnostics, "perturbation_l1", perturbation_l2)],
     [(pins_dg.test_perturbation_closed_form_and_full_budget_zero, ())]),
    ("weighted mass: head 0's weights", [(attention, "weighted_window_mass", weighted_mass_head0_weight)],
     [(pins_dg.test_weighted_window_mass, ())]),
    ("INT2: codes packed high bits first", [(int2, "pack_codes", pack_codes_reversed)],
     [(pins_int2.test_pack_bit_positions_hand_worked, ())]),
    ("fp16: round-down by nearest", [(fp, "f16_round_down", f16_round_down_by_nearest)],
     [(pins_int2.test_f16_directed_rounding_against_exhaustive_table, ())]),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_pins_catch_planted_mistake(case, monkeypatch):
    _, patches, pins = case
    for mod, attr, repl in patches:
        monkeypatch.setattr(mod, attr, repl)
    caught = [_fails(pin, *args) for pin, args in pins]
    assert any(caught), "no pin failed"


def test_pins_pass_on_the_oracle_as_written():
    """The same pins, unpatched (the cases above are meaningful only if these pass)."""
    for _, _, pins in CASES:
        for pin, args in pins:
            assert not _fails(pin, *args), pin.__name__

"""Writes the oracle regression fixtures in this folder. It calls only the oracle and the seeded input generators,
so the stored values are the oracle's own; the test that reads them fails if the oracle's arithmetic changes.

    python tests/golden/make_golden.py

Fixtures:
  tiny_decode_oracle.json  the tiny workload (two KV-head units, 1024 tokens, fp16), unit 0 through 8 decode steps
                           with routing after steps 4 and 8 (budgets 8 FULL / 8 INT2): the attention output of
                           heads 0 and 3 at steps 1 and 8 (first 8 head_dim entries), the cumulative scores after
                           step 8 (first 16 windows), the tiers after each event, the ledger's windows, and the
                           same run with span summaries: the summary count and the first summary's first 8 key
                           bits, and the output of head 0 at step 8.
"""
from __future__ import annotations

import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from kv_cache_compression_gqa_amd import configs, synth  # noqa: E402
from oracle.qevict import QEvictUnit  # noqa: E402


def tiny_run(summaries: bool):
    cfg = configs.TINY
    inp = synth.make_decode(cfg, units=[0], steps=8)
    nw, t0 = int(inp.n_windows[0]), int(inp.tail0[0])
    unit = QEvictUnit(inp.k_win[0, :nw], inp.v_win[0, :nw], inp.k_tail0[0, :t0], inp.v_tail0[0, :t0], cfg.dtype,
                      summaries=summaries)
    outs, tiers = {}, []
    for t in range(8):
        r = unit.step(inp.q[t, 0], inp.k_new[t, 0], inp.v_new[t, 0])
        if t in (0, 7):
            outs[t + 1] = r.o
        if (t + 1) % cfg.route_every == 0:
            unit.route(cfg.budget_full, cfg.budget_int2)
            tiers.append([int(x) for x in unit.tier])
    return unit, outs, tiers


def main():
    unit, outs, tiers = tiny_run(False)
    sunit, souts, _ = tiny_run(True)
    rec = {
        "source": "oracle/qevict.py and oracle/summary.py on kv_cache_compression_gqa_amd.synth.make_decode(TINY)",
        "out_step1_head0": [float(x) for x in outs[1][0, :8]],
        "out_step1_head3": [float(x) for x in outs[1][3, :8]],
        "out_step8_head0": [float(x) for x in outs[8][0, :8]],
        "cum_after_step8": [float(x) for x in unit.cum[:16]],
        "tiers_after_events": tiers,
        "ledger_windows": sorted(int(w) for w in unit.ledger),
        "summaries_count": len(sunit.sum_k),
        "first_summary_key_bits": [int(x) for x in sunit.sum_k[0][:8]],
        "summaries_out_step8_head0": [float(x) for x in souts[8][0, :8]],
    }
    with open(os.path.join(HERE, "tiny_decode_oracle.json"), "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()

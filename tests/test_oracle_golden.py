"""The oracle against its stored regression fixture (tests/golden/tiny_decode_oracle.json, written by
tests/golden/make_golden.py from the oracle itself): a change to the oracle's arithmetic shows up here and must be
justified by the passage it follows before the fixture is rewritten."""
import json
import os

import numpy as np

from tests.golden.make_golden import tiny_run

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_tiny_decode_matches_stored_oracle_values():
    rec = json.load(open(os.path.join(HERE, "tiny_decode_oracle.json")))
    unit, outs, tiers = tiny_run(False)
    assert np.allclose(outs[1][0, :8], rec["out_step1_head0"], rtol=1e-12, atol=0)
    assert np.allclose(outs[1][3, :8], rec["out_step1_head3"], rtol=1e-12, atol=0)
    assert np.allclose(outs[8][0, :8], rec["out_step8_head0"], rtol=1e-12, atol=0)
    assert np.allclose(unit.cum[:16], rec["cum_after_step8"], rtol=1e-12, atol=0)
    assert tiers == rec["tiers_after_events"]
    assert sorted(int(w) for w in unit.ledger) == rec["ledger_windows"]
    sunit, souts, _ = tiny_run(True)
    assert len(sunit.sum_k) == rec["summaries_count"]
    assert [int(x) for x in sunit.sum_k[0][:8]] == rec["first_summary_key_bits"]
    assert np.allclose(souts[8][0, :8], rec["summaries_out_step8_head0"], rtol=1e-12, atol=0)

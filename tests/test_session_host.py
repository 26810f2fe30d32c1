"""Host logic of the decode session, exercised on the CPU device (no library call is made)."""
import dataclasses

import numpy as np
import torch

from kv_cache_compression_gqa_amd import configs, synth
from kv_cache_compression_gqa_amd.session import DecodeSession


def test_session_state_and_bounds_on_cpu():
    for cfg in (configs.TINY, dataclasses.replace(configs.TINY, context=1000, name="r")):
        inp = synth.make_decode(cfg)
        s = DecodeSession(inp, device="cpu")
        NW = inp.n_windows_max
        assert s.k_full.shape == (2, NW, 32, 128) and s.FS == NW   # prefill pool: one slot per window
        bf, bq = cfg.budgets(int(inp.n_windows.max()))
        assert s.LS == min(NW, bf + bq) and s.k_codes.shape == (2, s.LS, 32, 32)
        assert s.FS_small == min(NW, max(1, bf)) and not s.repacked
        assert torch.equal(s.full_slot, s.res_list) and torch.equal(s.res_slot, s.res_list)
        assert torch.all(s.ledger_slot == -1)
        assert s.TM >= int(inp.tail0.max()) + cfg.steps + 1
        np.testing.assert_array_equal(s.k_tail[:, :int(inp.tail0.max())].numpy().view(np.uint16),
                                      inp.k_tail0[:, :int(inp.tail0.max())])
        assert s.bounds() == (int(inp.n_windows.max()), 0, int(inp.tail0.max()))
        a = s.decode_args(0)
        assert a.max_full == int(inp.n_windows.max()) and a.accumulate_cum == 1
        assert list(s.bf_host) == [cfg.budgets(int(n))[0] for n in inp.n_windows]
        assert torch.equal(s.res_list[0, :5], torch.arange(5, dtype=torch.int32))


def test_session_budget_bounds_follow_routing():
    inp = synth.make_decode(configs.LLAMA3_8B_LAYER_32K, units=[0, 1], steps=2)
    s = DecodeSession(inp, device="cpu")
    assert list(s.bf_host) == [204, 204] and list(s.bq_host) == [307, 307]
    # the host-side bound update a routing event applies
    n_res = s.h_full + s.h_int2
    nf = np.minimum(s.bf_host, n_res)
    nq = np.minimum(s.bq_host, n_res - nf)
    assert list(nf) == [204, 204] and list(nq) == [307, 307]
    # window memory: the prefill pool plus the pre-allocated b_full pool, then after the first event only the
    # b_full pool and the ledger pool (204 x 16 KiB + 511 x 3 KiB per unit)
    assert s.LS == 511 and s.FS_small == 204
    assert s.window_bytes() == 2 * (1024 + 204) * 16384 + 2 * 511 * 3072

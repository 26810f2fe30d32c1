"""kvc_decode_attn_static (the decode step with its scratch in the library's static device array, for callers
that cannot allocate) against kvc_decode_attn on the same inputs, through the C ABI: two sessions stepped side by
side, one per entry point, must agree bit for bit (same kernels, fixed reduction order) on the output, the
probabilities, the window mass, the cumulative score and the appended tail. Two workloads in a row, the second
smaller than the first, so the second call runs over what the first left in the array. A step needing more
scratch than the array holds is refused before any GPU work."""
import ctypes as C
import dataclasses
import sys

import numpy as np
import pytest
import torch

from kv_cache_compression_gqa_amd import abi, configs, synth
from kv_cache_compression_gqa_amd.session import DecodeSession

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _side_by_side(cfg, steps):
    inp = synth.make_decode(cfg, steps=steps)
    a, b = DecodeSession(inp), DecodeSession(inp)
    for t in range(steps):
        pa = torch.zeros((a.U, a.G, a.probs_stride()), dtype=torch.float32, device="cuda")
        pb = torch.zeros_like(pa)
        ma = torch.zeros((a.U, a.NW), dtype=torch.float32, device="cuda")
        mb = torch.zeros_like(ma)
        a.step(probs=pa, mass=ma)
        b.step(probs=pb, mass=mb, static_scratch=True)
        torch.cuda.synchronize()
        for name, x, y in (("out", a.out, b.out), ("probs", pa, pb), ("mass", ma, mb), ("cum", a.cum, b.cum),
                           ("tier", a.tier, b.tier), ("tail_len", a.tail_len, b.tail_len),
                           ("k_tail", a.k_tail, b.k_tail), ("v_tail", a.v_tail, b.v_tail)):
            assert torch.equal(x, y), f"{cfg.name} step {t}: {name} differs"
    assert a.device_status() == 0 and b.device_status() == 0


def test_static_scratch_matches_workspace_entry_point_two_calls(gpu_lib):
    big = dataclasses.replace(configs.LLAMA3_8B_LAYER_32K, name="static_8k", context=8192 + 21, steps=6,
                              route_every=3)
    small = dataclasses.replace(configs.TINY, name="static_tiny", steps=6, route_every=2)
    log(f"case: {big.name}, {big.n_units} units, 6 steps")
    _side_by_side(big, 6)
    log(f"case: {small.name}, {small.n_units} units, 6 steps (after the larger one)")
    _side_by_side(small, 6)


def test_static_scratch_refuses_oversized_steps(gpu_lib):
    cfg = dataclasses.replace(configs.TINY, name="static_big", layers=64, batch=32)
    inp = synth.make_decode(dataclasses.replace(cfg, layers=1, batch=1), steps=1)
    U = cfg.n_units // 2 * 2
    sess = DecodeSession(inp, unit_map=np.arange(U) % len(inp.units))
    args = sess.decode_args(0)
    L = abi.lib()
    need = L.kvc_decode_attn_workspace(C.byref(sess._cache), C.byref(args))
    assert need > L.kvc_decode_attn_static_max_bytes(), (need, U)
    before = sess.tail_len.clone()
    st = L.kvc_decode_attn_static(C.byref(sess._cache), C.byref(args), abi.stream_handle())
    torch.cuda.synchronize()
    assert st == abi.KVC_E_WORKSPACE
    assert torch.equal(sess.tail_len, before)   # nothing ran

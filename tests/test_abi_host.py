"""The C-ABI library loads on a machine without a GPU, exports every function include/kvc.h declares, and its
host-side validation rejects bad arguments before any GPU work (no compute call is made here)."""
import ctypes as C
import os
import re

import pytest

from kv_cache_compression_gqa_amd import abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if h.endswith(".h"):
            src = open(os.path.join(ROOT, "include", h)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(kvc_[a-z0-9_]+)\s*\(", src))
    return sorted(names)


def test_every_declared_symbol_is_exported_and_bound():
    L = abi.lib()
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n
        assert n in abi.SIGNATURES, n
    assert L.kvc_abi_version() == abi.ABI_VERSION == 6


def test_struct_sizes_match_header_layout():
    # 10 int32 + 20 pointers, then 3 pointers + 2 int32 for the span summaries
    assert C.sizeof(abi.KvcCache) == 10 * 4 + 20 * 8 + 3 * 8 + 2 * 4
    assert C.sizeof(abi.KvcDecodeArgs) == 6 * 8 + 6 * 4 + 2 * 8 + 2 * 4
    assert C.sizeof(abi.KvcTierRouteArgs) == 8 * 8


def test_status_strings():
    L = abi.lib()
    for st in range(-6, 1):
        assert len(L.kvc_status_str(st)) > 0


FAKE = 0x10000  # 64 KiB-aligned fake device address; validation fails before anything dereferences it


def good_cache(**over):
    kw = dict(n_units=2, group=4, head_dim=128, window=32, n_windows_max=32, tail_max=64, kv_dtype=abi.KVC_BF16,
              full_slots=32, ledger_slots=16, reserved=0)
    for f, _ in abi.KvcCache._fields_[10:]:
        kw[f] = FAKE
    kw.update(k_sum=None, v_sum=None, n_sum=None, sum_max=0, reserved2=0)   # no span summaries
    kw.update(over)
    return abi.KvcCache(**kw)


def good_step(**over):
    kw = dict(q=FAKE, k_new=FAKE, v_new=FAKE, out=FAKE, probs=None, mass=None, probs_stride=0, accumulate_cum=1,
              max_full=8, max_int2=8, max_tail=10, reserved=0)
    kw.update(over)
    return abi.KvcDecodeArgs(**kw)


@pytest.mark.parametrize("cache_over,step_over,status", [
    (dict(head_dim=64), {}, abi.KVC_E_UNSUPPORTED),
    (dict(window=16), {}, abi.KVC_E_UNSUPPORTED),
    (dict(group=3), {}, abi.KVC_E_UNSUPPORTED),
    (dict(kv_dtype=7), {}, abi.KVC_E_UNSUPPORTED),
    (dict(n_units=0), {}, abi.KVC_E_INVALID),
    (dict(k_full=None), {}, abi.KVC_E_INVALID),
    (dict(full_slot=None), {}, abi.KVC_E_INVALID),
    (dict(res_slot=FAKE + 2), {}, abi.KVC_E_INVALID),
    (dict(full_slots=0), {}, abi.KVC_E_INVALID),
    (dict(ledger_slots=-1), {}, abi.KVC_E_INVALID),
    (dict(k_tail=FAKE + 2), {}, abi.KVC_E_INVALID),
    ({}, dict(q=None), abi.KVC_E_INVALID),
    ({}, dict(v_new=None), abi.KVC_E_INVALID),
    ({}, dict(out=None), abi.KVC_E_INVALID),
    ({}, dict(max_full=-1), abi.KVC_E_BUDGET),
    ({}, dict(max_full=30, max_int2=8), abi.KVC_E_BUDGET),
    ({}, dict(max_tail=64), abi.KVC_E_BUDGET),
    ({}, dict(probs=FAKE, probs_stride=10), abi.KVC_E_INVALID),
    ({}, dict(accumulate_cum=2), abi.KVC_E_INVALID),
])
def test_decode_attn_validation(cache_over, step_over, status):
    L = abi.lib()
    c, s = good_cache(**cache_over), good_step(**step_over)
    assert L.kvc_decode_attn(C.byref(c), C.byref(s), FAKE, 1 << 30, None) == status


def test_decode_attn_static_validation_rejects_before_launch():
    """kvc_decode_attn_static validates like kvc_decode_attn and refuses a step whose scratch exceeds its static
    array (16 MiB) before touching the GPU."""
    L = abi.lib()
    assert L.kvc_decode_attn_static_max_bytes() == 16 << 20
    c, s = good_cache(head_dim=64), good_step()
    assert L.kvc_decode_attn_static(C.byref(c), C.byref(s), None) == abi.KVC_E_UNSUPPORTED
    assert L.kvc_decode_attn_static(C.byref(good_cache()), C.byref(good_step(q=None)), None) == abi.KVC_E_INVALID
    big = good_cache(n_units=4096, n_windows_max=256)
    sb = good_step(max_full=64, max_int2=64, max_tail=10)
    assert L.kvc_decode_attn_workspace(C.byref(big), C.byref(sb)) > 16 << 20
    assert L.kvc_decode_attn_static(C.byref(big), C.byref(sb), None) == abi.KVC_E_WORKSPACE


def test_decode_attn_workspace_checks():
    L = abi.lib()
    c, s = good_cache(), good_step()
    need = L.kvc_decode_attn_workspace(C.byref(c), C.byref(s))
    assert need > 0
    assert L.kvc_decode_attn(C.byref(c), C.byref(s), FAKE, need - 1, None) == abi.KVC_E_WORKSPACE
    assert L.kvc_decode_attn(C.byref(c), C.byref(s), None, need, None) == abi.KVC_E_WORKSPACE
    assert L.kvc_decode_attn(C.byref(c), C.byref(s), FAKE + 16, need, None) == abi.KVC_E_WORKSPACE
    assert L.kvc_decode_attn_workspace(C.byref(good_cache(head_dim=64)), C.byref(s)) == 0


def test_route_and_list_validation():
    L = abi.lib()
    c = good_cache()
    ra = abi.KvcTierRouteArgs(cache=C.pointer(c), scores=None, budget_full=FAKE, budget_int2=None,
                              quant_list=FAKE, n_quant=FAKE, promo_list=FAKE, n_promo=FAKE)
    assert L.kvc_route(abi.KVC_ROUTE_TIERS, C.byref(ra), None, 0, None) == abi.KVC_E_INVALID
    assert L.kvc_route(99, C.byref(ra), None, 0, None) == abi.KVC_E_UNSUPPORTED
    assert L.kvc_route(abi.KVC_ROUTE_TIERS, None, None, 0, None) == abi.KVC_E_INVALID
    assert L.kvc_quantize_int2(C.byref(c), FAKE, FAKE, 32, -1, None) == abi.KVC_E_BUDGET
    assert L.kvc_quantize_int2(C.byref(c), FAKE, FAKE, 32, 2 * 32 + 1, None) == abi.KVC_E_BUDGET
    assert L.kvc_quantize_int2(C.byref(c), None, FAKE, 32, 5, None) == abi.KVC_E_INVALID
    assert L.kvc_promote(C.byref(c), FAKE, FAKE, 0, 5, None) == abi.KVC_E_INVALID
    assert L.kvc_promote(C.byref(good_cache(window=8)), FAKE, FAKE, 32, 5, None) == abi.KVC_E_UNSUPPORTED
    # nothing to do is accepted without touching the device
    assert L.kvc_quantize_int2(C.byref(c), None, None, 32, 0, None) == abi.KVC_OK
    assert L.kvc_score(5, C.byref(ra), None, 0, None) == abi.KVC_E_UNSUPPORTED


def _status_of(fn, *args):
    return fn(*args)


def test_retention_topm_compact_validation_rejects_before_launch():
    L = abi.lib()
    # retention score: n_tokens must be a multiple of 4
    a = abi.KvcRetentionArgs(beta=FAKE, score=FAKE, n_rows=4, n_tokens=6, t=6)
    assert L.kvc_score(abi.KVC_SCORE_RETENTION, C.cast(C.byref(a), C.c_void_p), None, 0, None) == abi.KVC_E_INVALID
    a = abi.KvcRetentionArgs(beta=FAKE + 4, score=FAKE, n_rows=4, n_tokens=8, t=8)
    assert L.kvc_score(abi.KVC_SCORE_RETENTION, C.cast(C.byref(a), C.c_void_p), None, 0, None) == abi.KVC_E_INVALID
    # top-M: m outside [0, n], row length not a multiple of 16, missing workspace
    def topm(**over):
        kw = dict(scores=FAKE, n=64, m=8, row_len=32, reserved=0, keep=FAKE, row_counts=FAKE, status=FAKE, beta=None,
                  t=64, reserved2=0)
        kw.update(over)
        t = abi.KvcTopmArgs(**kw)
        return L.kvc_route(abi.KVC_ROUTE_GLOBAL_TOPM, C.cast(C.byref(t), C.c_void_p), None, 0, None), t
    assert topm(m=65)[0] == abi.KVC_E_BUDGET
    assert topm(m=-1)[0] == abi.KVC_E_BUDGET
    assert topm(row_len=24, n=48)[0] == abi.KVC_E_INVALID
    assert topm(n=50)[0] == abi.KVC_E_INVALID
    assert topm(beta=FAKE)[0] == abi.KVC_E_INVALID                 # scores and beta both given
    assert topm(scores=None)[0] == abi.KVC_E_INVALID               # neither
    assert topm(scores=None, beta=FAKE + 4)[0] == abi.KVC_E_INVALID
    assert topm(scores=None, beta=FAKE)[0] == abi.KVC_E_WORKSPACE  # fused input accepted (no workspace given)
    assert topm(reserved2=1)[0] == abi.KVC_E_INVALID
    # sizes whose per-row block count would overflow int32 arithmetic are refused
    big = (1 << 31) - 8192   # one past the largest supported n (2^31 - 8208, a multiple of 16)
    assert topm(n=big, row_len=big, m=1)[0] == abi.KVC_E_UNSUPPORTED
    assert topm(n=big - 16, row_len=big - 16, m=1)[0] != abi.KVC_E_UNSUPPORTED
    assert topm()[0] == abi.KVC_E_WORKSPACE
    st, t = topm()
    assert L.kvc_route_workspace(abi.KVC_ROUTE_GLOBAL_TOPM, C.cast(C.byref(t), C.c_void_p)) > 0
    # compaction: head_dim other than 128, page not dividing the row, missing workspace
    def compact(**over):
        kw = dict(keep=FAKE, page_table=FAKE, k_pool=FAKE, v_pool=FAKE, k_out=FAKE, v_out=FAKE, lengths=FAKE,
                  page_offset=FAKE, n_pages=FAKE, status=FAKE, n_rows=4, n_src_pages=16, out_pages_max=16,
                  n_tokens=64, page=16, head_dim=128, kv_dtype=abi.KVC_BF16)
        kw.update(over)
        c = abi.KvcCompactArgs(**kw)
        return L.kvc_compact_pages(C.byref(c), None, 0, None), c
    assert compact(head_dim=64)[0] == abi.KVC_E_UNSUPPORTED
    assert compact(page=24)[0] == abi.KVC_E_INVALID
    assert compact(kv_dtype=7)[0] == abi.KVC_E_UNSUPPORTED
    assert compact()[0] == abi.KVC_E_WORKSPACE
    assert L.kvc_compact_pages_workspace(C.byref(compact()[1])) > 0


def test_criticalkv_and_two_stage_validation_rejects_before_launch():
    L = abi.lib()

    def ckv(**over):
        kw = dict(q_obs=FAKE, k=FAKE, v=FAKE, w_o=FAKE, a_head=FAKE, norm=FAKE, a_group=FAKE, s2_group=FAKE,
                  n_keys=1024, hq=8, hkv=2, n_obs=32, head_dim=128, d_model=256, kv_dtype=abi.KVC_BF16, reserved=0)
        kw.update(over)
        c = abi.KvcCriticalKVArgs(**kw)
        pc = C.cast(C.byref(c), C.c_void_p)
        return L.kvc_score(abi.KVC_SCORE_CRITICALKV, pc, None, 0, None), L.kvc_score_workspace(abi.KVC_SCORE_CRITICALKV, pc)
    assert ckv(n_obs=16)[0] == abi.KVC_E_UNSUPPORTED
    assert ckv(hq=6)[0] == abi.KVC_E_UNSUPPORTED
    assert ckv(d_model=100)[0] == abi.KVC_E_UNSUPPORTED
    assert ckv(kv_dtype=5)[0] == abi.KVC_E_UNSUPPORTED
    assert ckv(reserved=1)[0] == abi.KVC_E_INVALID
    st, ws = ckv()
    assert st == abi.KVC_E_WORKSPACE and ws >= 8 * 256 * 128 * 2

    def ts(**over):
        kw = dict(a=FAKE, s2=FAKE, idx=FAKE, rows=2, n=100, budget=10, reserved=0, alpha=0.5)
        kw.update(over)
        t = abi.KvcTwoStageArgs(**kw)
        pa = C.cast(C.byref(t), C.c_void_p)
        return L.kvc_route(abi.KVC_ROUTE_TWO_STAGE, pa, FAKE, L.kvc_route_workspace(abi.KVC_ROUTE_TWO_STAGE, pa),
                           None)
    assert ts(budget=101) == abi.KVC_E_BUDGET
    assert ts(alpha=1.5) == abi.KVC_E_BUDGET
    assert ts(alpha=-0.1) == abi.KVC_E_BUDGET
    assert ts(alpha=float("nan")) == abi.KVC_E_BUDGET
    assert ts(reserved=1) == abi.KVC_E_INVALID
    assert ts(n=70000, budget=10) == abi.KVC_E_UNSUPPORTED
    assert ts(budget=0) == abi.KVC_OK  # nothing to select: no launch
    t = abi.KvcTwoStageArgs(a=FAKE, s2=FAKE, idx=FAKE, rows=2, n=100, budget=10, reserved=0, alpha=0.5)
    pa = C.cast(C.byref(t), C.c_void_p)
    need = L.kvc_route_workspace(abi.KVC_ROUTE_TWO_STAGE, pa)
    assert need > 0
    assert L.kvc_route(abi.KVC_ROUTE_TWO_STAGE, pa, None, need, None) == abi.KVC_E_WORKSPACE
    assert L.kvc_route(abi.KVC_ROUTE_TWO_STAGE, pa, FAKE, need - 1, None) == abi.KVC_E_WORKSPACE


def test_route_diagnostics_validation_rejects_before_launch():
    L = abi.lib()
    assert C.sizeof(abi.KvcDiagArgs) == 8 * 8 + 4 * 4

    def args(**over):
        kw = dict(tier_prev=FAKE, tier=FAKE, n_windows=FAKE, mass_full=FAKE, o_full=FAKE, o=FAKE, counts=FAKE,
                  values=FAKE, n_units=4, n_windows_max=32, group=4, head_dim=128)
        kw.update(over)
        return abi.KvcDiagArgs(**kw)

    assert L.kvc_route_diagnostics(None, None) == abi.KVC_E_INVALID
    assert L.kvc_route_diagnostics(C.byref(args(head_dim=64)), None) == abi.KVC_E_UNSUPPORTED
    assert L.kvc_route_diagnostics(C.byref(args(group=3)), None) == abi.KVC_E_UNSUPPORTED
    assert L.kvc_route_diagnostics(C.byref(args(n_units=0)), None) == abi.KVC_E_INVALID
    assert L.kvc_route_diagnostics(C.byref(args(n_windows_max=0)), None) == abi.KVC_E_INVALID
    assert L.kvc_route_diagnostics(C.byref(args(tier=None)), None) == abi.KVC_E_INVALID
    assert L.kvc_route_diagnostics(C.byref(args(counts=None)), None) == abi.KVC_E_INVALID
    assert L.kvc_route_diagnostics(C.byref(args(values=None)), None) == abi.KVC_E_INVALID
    assert L.kvc_route_diagnostics(C.byref(args(mass_full=FAKE + 2)), None) == abi.KVC_E_INVALID


def test_summary_validation_rejects_before_launch():
    L = abi.lib()
    # the cache's summary fields: all or nothing, capacity a multiple of 32
    assert L.kvc_decode_attn_workspace(C.byref(good_cache(k_sum=FAKE)), C.byref(good_step())) == 0
    assert L.kvc_decode_attn_workspace(C.byref(good_cache(sum_max=32)), C.byref(good_step())) == 0
    assert L.kvc_decode_attn_workspace(C.byref(good_cache(reserved2=1)), C.byref(good_step())) == 0
    with_sum = dict(k_sum=FAKE, v_sum=FAKE, n_sum=FAKE, sum_max=64)
    assert L.kvc_decode_attn_workspace(C.byref(good_cache(**with_sum, )), C.byref(good_step())) > 0
    assert L.kvc_decode_attn_workspace(C.byref(good_cache(k_sum=FAKE, v_sum=FAKE, n_sum=FAKE, sum_max=48)),
                                       C.byref(good_step())) == 0
    # a step that attends summaries needs them in the cache, within the capacity, and no probabilities
    c, s = good_cache(), good_step(max_summary=32)
    assert L.kvc_decode_attn(C.byref(c), C.byref(s), FAKE, 1 << 30, None) == abi.KVC_E_BUDGET
    c, s = good_cache(**with_sum), good_step(max_summary=96)
    assert L.kvc_decode_attn(C.byref(c), C.byref(s), FAKE, 1 << 30, None) == abi.KVC_E_BUDGET
    s = good_step(max_summary=32, probs=FAKE, probs_stride=1024)
    assert L.kvc_decode_attn(C.byref(c), C.byref(s), FAKE, 1 << 30, None) == abi.KVC_E_UNSUPPORTED
    s = good_step(max_summary=-1)
    assert L.kvc_decode_attn(C.byref(c), C.byref(s), FAKE, 1 << 30, None) == abi.KVC_E_INVALID
    # kvc_summarize_evicted
    need = L.kvc_summarize_workspace(C.byref(c))
    assert need > 0 and L.kvc_summarize_workspace(None) == 0
    assert L.kvc_summarize_evicted(None, FAKE, 1, FAKE, need, None) == abi.KVC_E_INVALID
    assert L.kvc_summarize_evicted(C.byref(good_cache()), FAKE, 1, FAKE, need, None) == abi.KVC_E_INVALID
    assert L.kvc_summarize_evicted(C.byref(c), None, 1, FAKE, need, None) == abi.KVC_E_INVALID
    assert L.kvc_summarize_evicted(C.byref(c), FAKE, 33, FAKE, need, None) == abi.KVC_E_INVALID   # > NW
    assert L.kvc_summarize_evicted(C.byref(c), FAKE, -1, FAKE, need, None) == abi.KVC_E_INVALID
    assert L.kvc_summarize_evicted(C.byref(c), FAKE, 1, FAKE, need - 1, None) == abi.KVC_E_WORKSPACE
    assert L.kvc_summarize_evicted(C.byref(c), FAKE, 1, FAKE + 16, need, None) == abi.KVC_E_WORKSPACE


def test_token_weight_validation_rejects_before_launch():
    L = abi.lib()
    c = good_cache()
    s = good_step(token_weight=FAKE, weight_stride=32 * 32 - 1)   # below n_windows_max * W
    assert L.kvc_decode_attn(C.byref(c), C.byref(s), FAKE, 1 << 30, None) == abi.KVC_E_INVALID
    s = good_step(token_weight=FAKE + 2, weight_stride=32 * 32)
    assert L.kvc_decode_attn(C.byref(c), C.byref(s), FAKE, 1 << 30, None) == abi.KVC_E_INVALID


def test_header_is_plain_c_and_links(tmp_path):
    """include/kvc.h and include/kvc_probe.h compile as C99 with warnings as errors, and a C program links against the library and sees
    the same ABI version the header states."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    src = tmp_path / "kvc_check.c"
    src.write_text('#include "kvc.h"\n'
                   '#include "kvc_probe.h"\n'
                   "int main(void) {\n"
                   "  kvc_cache c; kvc_decode_args a; kvc_diag_args d; (void)c; (void)a; (void)d;\n"
                   "  if (kvc_probe_stream_workgroups(3) != 3) return 2;\n"
                   "  return kvc_abi_version() == KVC_ABI_VERSION ? 0 : 1;\n"
                   "}\n")
    lib_dir = os.path.dirname(abi.lib_path())
    exe = tmp_path / "kvc_check"
    r = subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                        "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", str(src), "-L", lib_dir,
                        "-lkvc", f"-Wl,-rpath,{lib_dir}", "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    assert subprocess.run([str(exe)]).returncode == 0


def test_probe_validation_rejects_before_launch():
    L = abi.lib()
    assert L.kvc_probe_stream_workgroups(-1) == 0 and L.kvc_probe_stream_workgroups(12) == 12
    assert L.kvc_probe_stream_read(None, 1024, 0, FAKE, None) == abi.KVC_E_INVALID
    assert L.kvc_probe_stream_read(FAKE + 4, 1024, 0, FAKE, None) == abi.KVC_E_INVALID
    assert L.kvc_probe_stream_read(FAKE, 1000, 0, FAKE, None) == abi.KVC_E_INVALID
    assert L.kvc_probe_stream_read(FAKE, 1 << 41, 0, FAKE, None) == abi.KVC_E_UNSUPPORTED
    assert L.kvc_probe_wave_read(FAKE, 1000, FAKE, None) == abi.KVC_E_INVALID
    assert L.kvc_probe_wave_read(FAKE, 16384, None, None) == abi.KVC_E_INVALID
    assert L.kvc_probe_wave_read(FAKE, 0, FAKE, None) == abi.KVC_OK


def test_topk_validation_rejects_before_launch():
    L = abi.lib()
    assert L.kvc_topk_workspace(-1, 0) == 0 and L.kvc_topk_workspace(10, 11) == 0
    assert L.kvc_topk_workspace(10, -1) == 0 and L.kvc_topk_workspace(1 << 31, 1) == 0
    need = L.kvc_topk_workspace(1000, 10)
    assert need > 0
    assert L.kvc_topk(FAKE, 1000, 0, None, None, 0, None) == abi.KVC_OK          # nothing to select
    assert L.kvc_topk(FAKE, 1000, 1001, FAKE, FAKE, need, None) == abi.KVC_E_BUDGET
    assert L.kvc_topk(FAKE, -1, 1, FAKE, FAKE, need, None) == abi.KVC_E_INVALID
    assert L.kvc_topk(FAKE, 1 << 31, 1, FAKE, FAKE, need, None) == abi.KVC_E_UNSUPPORTED
    limit = (1 << 31) - 8208
    assert L.kvc_topk_workspace(limit + 1, 1) == 0 and L.kvc_topk_workspace(limit, 1) > 0
    assert L.kvc_topk(FAKE, limit + 1, 1, FAKE, FAKE, need, None) == abi.KVC_E_UNSUPPORTED
    assert L.kvc_topk(None, 1000, 10, FAKE, FAKE, need, None) == abi.KVC_E_INVALID
    assert L.kvc_topk(FAKE + 4, 1000, 10, FAKE, FAKE, need, None) == abi.KVC_E_INVALID
    assert L.kvc_topk(FAKE, 1000, 10, None, FAKE, need, None) == abi.KVC_E_INVALID
    assert L.kvc_topk(FAKE, 1000, 10, FAKE, FAKE, need - 1, None) == abi.KVC_E_WORKSPACE
    assert L.kvc_topk(FAKE, 1000, 10, FAKE, FAKE + 16, need, None) == abi.KVC_E_WORKSPACE

"""ctypes binding of the C ABI in include/kvc.h (argument marshalling only; all work runs in the HIP library).

The library is loaded from ``kv_cache_compression_gqa_amd/lib/libkvc.so`` (built in-tree by
``kv_cache_compression_gqa_amd.build``). If it is missing, every call raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libkvc.so")
_lib = None

ABI_VERSION = 6  # KVC_ABI_VERSION of include/kvc.h
KVC_OK, KVC_E_INVALID, KVC_E_UNSUPPORTED, KVC_E_WORKSPACE, KVC_E_LEDGER, KVC_E_BUDGET, KVC_E_HIP = \
    0, -1, -2, -3, -4, -5, -6
KVC_DEV_LEDGER_REWRITE, KVC_DEV_BOUND_EXCEEDED, KVC_DEV_NAN_SCORE = 0x1, 0x2, 0x4
KVC_F16, KVC_BF16 = 0, 1
TIER_FULL, TIER_INT2, TIER_EVICTED = 0, 1, 2
KVC_SCORE_WINDOWS, KVC_SCORE_RETENTION, KVC_SCORE_CRITICALKV = 0, 1, 2
KVC_ROUTE_TIERS, KVC_ROUTE_GLOBAL_TOPM, KVC_ROUTE_TWO_STAGE = 0, 1, 2

P = C.c_void_p


class KvcError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        msg = lib().kvc_status_str(status).decode() if _lib is not None else str(status)
        super().__init__(f"{what}: kvc status {status} ({msg})")


class KvcCache(C.Structure):
    _fields_ = [("n_units", C.c_int32), ("group", C.c_int32), ("head_dim", C.c_int32), ("window", C.c_int32),
                ("n_windows_max", C.c_int32), ("tail_max", C.c_int32), ("kv_dtype", C.c_int32),
                ("full_slots", C.c_int32), ("ledger_slots", C.c_int32), ("reserved", C.c_int32),
                ("n_windows", P), ("k_full", P), ("v_full", P), ("k_codes", P), ("v_codes", P), ("k_meta", P),
                ("v_meta", P), ("k_tail", P), ("v_tail", P), ("tail_len", P), ("tier", P), ("ledgered", P),
                ("full_slot", P), ("ledger_slot", P), ("cum", P), ("res_list", P), ("res_slot", P), ("n_full", P),
                ("n_int2", P), ("status", P), ("k_sum", P), ("v_sum", P), ("n_sum", P), ("sum_max", C.c_int32),
                ("reserved2", C.c_int32)]


class KvcDecodeArgs(C.Structure):
    _fields_ = [("q", P), ("k_new", P), ("v_new", P), ("out", P), ("probs", P), ("mass", P),
                ("probs_stride", C.c_int32), ("accumulate_cum", C.c_int32), ("max_full", C.c_int32),
                ("max_int2", C.c_int32), ("max_tail", C.c_int32), ("reserved", C.c_int32), ("token_weight", P),
                ("weight_stride", C.c_int64), ("max_summary", C.c_int32), ("reserved2", C.c_int32)]


class KvcTierRouteArgs(C.Structure):
    _fields_ = [("cache", C.POINTER(KvcCache)), ("scores", P), ("budget_full", P), ("budget_int2", P),
                ("quant_list", P), ("n_quant", P), ("promo_list", P), ("n_promo", P)]


class KvcWindowScoreArgs(C.Structure):
    _fields_ = [("cache", C.POINTER(KvcCache)), ("step", C.POINTER(KvcDecodeArgs))]


class KvcRetentionArgs(C.Structure):
    _fields_ = [("beta", P), ("score", P), ("n_rows", C.c_int64), ("n_tokens", C.c_int32), ("t", C.c_int32)]


class KvcTopmArgs(C.Structure):
    _fields_ = [("scores", P), ("n", C.c_int64), ("m", C.c_int64), ("row_len", C.c_int32), ("reserved", C.c_int32),
                ("keep", P), ("row_counts", P), ("status", P), ("beta", P), ("t", C.c_int32), ("reserved2", C.c_int32)]


class KvcCompactArgs(C.Structure):
    _fields_ = [("keep", P), ("page_table", P), ("k_pool", P), ("v_pool", P), ("k_out", P), ("v_out", P),
                ("lengths", P), ("page_offset", P), ("n_pages", P), ("status", P), ("n_rows", C.c_int64),
                ("n_src_pages", C.c_int64), ("out_pages_max", C.c_int64), ("n_tokens", C.c_int32),
                ("page", C.c_int32), ("head_dim", C.c_int32), ("kv_dtype", C.c_int32)]


class KvcCriticalKVArgs(C.Structure):
    _fields_ = [("q_obs", P), ("k", P), ("v", P), ("w_o", P), ("a_head", P), ("norm", P), ("a_group", P),
                ("s2_group", P), ("n_keys", C.c_int32), ("hq", C.c_int32), ("hkv", C.c_int32), ("n_obs", C.c_int32),
                ("head_dim", C.c_int32), ("d_model", C.c_int32), ("kv_dtype", C.c_int32), ("reserved", C.c_int32)]


class KvcTwoStageArgs(C.Structure):
    _fields_ = [("a", P), ("s2", P), ("idx", P), ("rows", C.c_int32), ("n", C.c_int32), ("budget", C.c_int32),
                ("reserved", C.c_int32), ("alpha", C.c_double)]


class KvcPagedDecodeArgs(C.Structure):
    _fields_ = [("q", P), ("k_pool", P), ("v_pool", P), ("page_list", P), ("lengths", P), ("out", P), ("status", P),
                ("n_rows", C.c_int64), ("n_pool_pages", C.c_int64), ("page_stride", C.c_int64),
                ("group", C.c_int32), ("page", C.c_int32), ("max_pages", C.c_int32), ("head_dim", C.c_int32),
                ("kv_dtype", C.c_int32), ("reserved", C.c_int32)]


class KvcDiagArgs(C.Structure):
    _fields_ = [("tier_prev", P), ("tier", P), ("n_windows", P), ("mass_full", P), ("o_full", P), ("o", P),
                ("counts", P), ("values", P), ("n_units", C.c_int32), ("n_windows_max", C.c_int32),
                ("group", C.c_int32), ("head_dim", C.c_int32)]


# name -> (restype, argtypes); every symbol include/kvc.h and include/kvc_probe.h declare
SIGNATURES = {
    "kvc_probe_stream_workgroups": (C.c_int, [C.c_int32]),
    "kvc_probe_stream_read": (C.c_int, [P, C.c_size_t, C.c_int32, P, P]),
    "kvc_probe_wave_read": (C.c_int, [P, C.c_size_t, P, P]),
    "kvc_abi_version": (C.c_int, []),
    "kvc_status_str": (C.c_char_p, [C.c_int]),
    "kvc_decode_attn_workspace": (C.c_size_t, [C.POINTER(KvcCache), C.POINTER(KvcDecodeArgs)]),
    "kvc_decode_attn": (C.c_int, [C.POINTER(KvcCache), C.POINTER(KvcDecodeArgs), P, C.c_size_t, P]),
    "kvc_decode_attn_static": (C.c_int, [C.POINTER(KvcCache), C.POINTER(KvcDecodeArgs), P]),
    "kvc_decode_attn_static_max_bytes": (C.c_size_t, []),
    "kvc_score_workspace": (C.c_size_t, [C.c_int32, P]),
    "kvc_score": (C.c_int, [C.c_int32, P, P, C.c_size_t, P]),
    "kvc_route_workspace": (C.c_size_t, [C.c_int32, P]),
    "kvc_route": (C.c_int, [C.c_int32, P, P, C.c_size_t, P]),
    "kvc_quantize_int2": (C.c_int, [C.POINTER(KvcCache), P, P, C.c_int32, C.c_int64, P]),
    "kvc_promote": (C.c_int, [C.POINTER(KvcCache), P, P, C.c_int32, C.c_int64, P]),
    "kvc_read_device_status": (C.c_int, [C.POINTER(KvcCache), C.POINTER(C.c_int32), C.c_int32, P]),
    "kvc_compact_pages_workspace": (C.c_size_t, [C.POINTER(KvcCompactArgs)]),
    "kvc_compact_pages": (C.c_int, [C.POINTER(KvcCompactArgs), P, C.c_size_t, P]),
    "kvc_paged_decode_workspace": (C.c_size_t, [C.POINTER(KvcPagedDecodeArgs)]),
    "kvc_paged_decode_attn": (C.c_int, [C.POINTER(KvcPagedDecodeArgs), P, C.c_size_t, P]),
    "kvc_route_diagnostics": (C.c_int, [C.POINTER(KvcDiagArgs), P]),
    "kvc_summarize_workspace": (C.c_size_t, [C.POINTER(KvcCache)]),
    "kvc_topk_workspace": (C.c_size_t, [C.c_int64, C.c_int64]),
    "kvc_topk": (C.c_int, [P, C.c_int64, C.c_int64, P, P, C.c_size_t, P]),
    "kvc_summarize_evicted": (C.c_int, [C.POINTER(KvcCache), P, C.c_int32, P, C.c_size_t, P]),
    "kvc_repack_full": (C.c_int, [C.POINTER(KvcCache), P, P, C.c_int32, P]),
}


def lib_path() -> str:
    return _LIB_PATH


def lib():
    """Load (once) and return the HIP library. Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"HIP library not built: {_LIB_PATH} is missing "
                               "(run `python -m kv_cache_compression_gqa_amd.build`)")
        L = C.CDLL(_LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        if L.kvc_abi_version() != ABI_VERSION:
            raise RuntimeError("kvc ABI version mismatch")
        _lib = L
    return _lib


def check(status: int, what: str):
    if status != KVC_OK:
        raise KvcError(status, what)


def ptr(t) -> int | None:
    """Device pointer of a torch tensor (or None)."""
    return None if t is None else t.data_ptr()


def stream_handle(stream=None) -> int:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream

"""CriticalKV prefill scores and two-stage selection on the GPU.

CriticalKV page ("Resumo Técnico: CriticalKV"), "Framework Teórico" and "Algoritmo: Seleção Constrainda por
Perturbação". Thin wrappers over kvc_score(CRITICALKV) and kvc_route(TWO_STAGE): torch tensors in, argument
marshalling only.
"""
from __future__ import annotations

import ctypes as C

import torch

from . import abi


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def scores(q_obs: torch.Tensor, k: torch.Tensor, v: torch.Tensor, w_o: torch.Tensor, kv_dtype: int, stream=None):
    """q_obs [Hq][32][128], k, v [Hkv][n][128], w_o [Hq*128][d_model] (16-bit storage, cuda) ->
    dict of float32 tensors: a_head, norm [Hq][n]; a_group, s2_group [Hkv][n]."""
    hq, n_obs, D = q_obs.shape
    hkv, n, _ = k.shape
    dm = w_o.shape[1]
    dev = k.device
    out = {name: torch.empty(shape, dtype=torch.float32, device=dev)
           for name, shape in (("a_head", (hq, n)), ("norm", (hq, n)), ("a_group", (hkv, n)), ("s2_group", (hkv, n)))}
    a = abi.KvcCriticalKVArgs(q_obs=q_obs.data_ptr(), k=k.data_ptr(), v=v.data_ptr(), w_o=w_o.data_ptr(),
                              a_head=out["a_head"].data_ptr(), norm=out["norm"].data_ptr(),
                              a_group=out["a_group"].data_ptr(), s2_group=out["s2_group"].data_ptr(), n_keys=n,
                              hq=hq, hkv=hkv, n_obs=n_obs, head_dim=D, d_model=dm, kv_dtype=kv_dtype, reserved=0)
    L = abi.lib()
    pa = C.cast(C.byref(a), C.c_void_p)
    need = L.kvc_score_workspace(abi.KVC_SCORE_CRITICALKV, pa)
    if need == 0:
        raise abi.KvcError(abi.KVC_E_INVALID, "kvc_score_workspace(CRITICALKV)")
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    abi.check(L.kvc_score(abi.KVC_SCORE_CRITICALKV, pa, ws.data_ptr(), need, _stream(stream)), "kvc_score(CRITICALKV)")
    out["_ws"] = ws
    return out


def two_stage(a: torch.Tensor, s2: torch.Tensor, budget: int, alpha: float, stream=None, workspace=None):
    """a, s2 [rows][n] float32 (cuda) -> [rows][budget] int32 ascending: first floor(alpha*budget) by a, the rest
    by s2 among the entries not yet taken; ties to the lower index (the library takes the floor)."""
    rows, n = a.shape
    idx = torch.empty((rows, budget), dtype=torch.int32, device=a.device)
    args = abi.KvcTwoStageArgs(a=a.data_ptr(), s2=s2.data_ptr(), idx=idx.data_ptr(), rows=rows, n=n, budget=budget,
                               reserved=0, alpha=float(alpha))
    L = abi.lib()
    pa = C.cast(C.byref(args), C.c_void_p)
    need = L.kvc_route_workspace(abi.KVC_ROUTE_TWO_STAGE, pa)
    if need == 0 and rows > 0 and budget > 0:
        raise abi.KvcError(abi.KVC_E_INVALID, "kvc_route_workspace(TWO_STAGE)")
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=a.device)
    abi.check(L.kvc_route(abi.KVC_ROUTE_TWO_STAGE, pa, workspace.data_ptr(), workspace.numel(), _stream(stream)),
              "kvc_route(TWO_STAGE)")
    return idx

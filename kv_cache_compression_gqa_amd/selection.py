"""Generic budgeted top-k on the GPU (kvc_topk): torch tensors in, argument marshalling only."""
from __future__ import annotations

import ctypes as C

import torch

from . import abi


def topk(scores: torch.Tensor, k: int, stream=None) -> torch.Tensor:
    """scores [n] float32 (cuda, contiguous) -> the indices of the first k entries in the order (score desc,
    index asc), ascending, int32 [k]."""
    assert scores.is_cuda and scores.dtype == torch.float32 and scores.dim() == 1 and scores.is_contiguous()
    n = scores.numel()
    out = torch.empty(k, dtype=torch.int32, device=scores.device)
    L = abi.lib()
    need = L.kvc_topk_workspace(n, k)
    if need == 0:
        raise abi.KvcError(abi.KVC_E_INVALID, "kvc_topk_workspace")
    ws = torch.empty(need, dtype=torch.uint8, device=scores.device)
    s = stream if stream is not None else torch.cuda.current_stream()
    abi.check(L.kvc_topk(scores.data_ptr(), n, k, out.data_ptr() if k > 0 else None, ws.data_ptr(), need,
                         C.c_void_p(s.cuda_stream)), "kvc_topk")
    out.ws = ws  # keep alive until the stream reaches the work
    return out

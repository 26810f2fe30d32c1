"""Global retention budget on the GPU: log-retention scores, one global top-M, per-row paged compaction.

DBTrimKV page ("Make Each Token Count: Towards Improving Long-Context Performance with KV Cache Eviction"),
"Metodologia: Evicção Baseada em Retenção Global", sections 2-4. Thin wrappers over kvc_score(RETENTION),
kvc_route(GLOBAL_TOPM), kvc_compact_pages and kvc_paged_decode_attn (decoding over the per-row page lists):
torch tensors in, argument marshalling only.
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass

import torch

from . import abi


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def retention_scores(beta: torch.Tensor, t: int, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """beta [rows][n_tokens] float32 (cuda) -> score = (t - i) * ln(beta), float32."""
    assert beta.is_cuda and beta.dtype == torch.float32 and beta.is_contiguous() and beta.dim() == 2
    out = torch.empty_like(beta) if out is None else out
    a = abi.KvcRetentionArgs(beta=beta.data_ptr(), score=out.data_ptr(), n_rows=beta.shape[0],
                             n_tokens=beta.shape[1], t=int(t))
    abi.check(abi.lib().kvc_score(abi.KVC_SCORE_RETENTION, C.cast(C.byref(a), C.c_void_p), None, 0, _stream(stream)),
              "kvc_score(RETENTION)")
    return out


@dataclass
class TopM:
    keep: torch.Tensor        # [rows][row_len] uint8
    row_counts: torch.Tensor  # [rows] int32
    status: torch.Tensor      # [1] int32


def global_topm(scores: torch.Tensor | None, m: int, stream=None, beta: torch.Tensor | None = None,
                t: int | None = None, workspace: torch.Tensor | None = None) -> TopM:
    """scores [rows][row_len] float32 (cuda) -> keep mask of the first m entries in (score desc, flat asc) order.
    With ``scores`` None, ``beta`` [rows][row_len] and ``t``: the scores are the log-retention (t - i) ln(beta),
    computed by the kernels where they are used (never written). ``workspace``: a uint8 tensor to reuse if large
    enough."""
    src = scores if scores is not None else beta
    assert src is not None and (scores is None) != (beta is None)
    assert src.is_cuda and src.dtype == torch.float32 and src.is_contiguous() and src.dim() == 2
    rows, row_len = src.shape
    dev = src.device
    res = TopM(keep=torch.empty((rows, row_len), dtype=torch.uint8, device=dev),
               row_counts=torch.empty(rows, dtype=torch.int32, device=dev),
               status=torch.zeros(1, dtype=torch.int32, device=dev))
    a = abi.KvcTopmArgs(scores=abi.ptr(scores), n=rows * row_len, m=int(m), row_len=row_len, reserved=0,
                        keep=res.keep.data_ptr(), row_counts=res.row_counts.data_ptr(),
                        status=res.status.data_ptr(), beta=abi.ptr(beta), t=int(t or 0), reserved2=0)
    L = abi.lib()
    pa = C.cast(C.byref(a), C.c_void_p)
    need = L.kvc_route_workspace(abi.KVC_ROUTE_GLOBAL_TOPM, pa)
    if need == 0:
        raise abi.KvcError(abi.KVC_E_INVALID, "kvc_route_workspace(GLOBAL_TOPM)")
    ws = workspace if workspace is not None and workspace.numel() >= need else \
        torch.empty(need, dtype=torch.uint8, device=dev)
    abi.check(L.kvc_route(abi.KVC_ROUTE_GLOBAL_TOPM, pa, ws.data_ptr(), ws.numel(), _stream(stream)),
              "kvc_route(GLOBAL_TOPM)")
    res.ws = ws  # keep alive until the stream reaches the work
    return res


@dataclass
class Compacted:
    k: torch.Tensor            # [out_pages_max][page][D]
    v: torch.Tensor
    lengths: torch.Tensor      # [rows] int32
    page_offset: torch.Tensor  # [rows] int32
    n_pages: torch.Tensor      # [rows] int32
    status: torch.Tensor       # [1] int32


def compact_pages(keep: torch.Tensor, page_table: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                  out_pages_max: int, kv_dtype: int, stream=None) -> Compacted:
    """keep [rows][T] uint8, page_table [rows][T/page] int32, pools [src_pages][page][D] (16-bit storage) ->
    the kept rows of every row copied, in order, into fresh pages (row r owns pages page_offset[r] ..)."""
    rows, T = keep.shape
    n_src, page, D = k_pool.shape
    dev = keep.device
    out = Compacted(k=torch.empty((out_pages_max, page, D), dtype=k_pool.dtype, device=dev),
                    v=torch.empty((out_pages_max, page, D), dtype=v_pool.dtype, device=dev),
                    lengths=torch.empty(rows, dtype=torch.int32, device=dev),
                    page_offset=torch.empty(rows, dtype=torch.int32, device=dev),
                    n_pages=torch.empty(rows, dtype=torch.int32, device=dev),
                    status=torch.zeros(1, dtype=torch.int32, device=dev))
    a = abi.KvcCompactArgs(keep=keep.data_ptr(), page_table=page_table.data_ptr(), k_pool=k_pool.data_ptr(),
                           v_pool=v_pool.data_ptr(), k_out=out.k.data_ptr(), v_out=out.v.data_ptr(),
                           lengths=out.lengths.data_ptr(), page_offset=out.page_offset.data_ptr(),
                           n_pages=out.n_pages.data_ptr(), status=out.status.data_ptr(), n_rows=rows,
                           n_src_pages=n_src, out_pages_max=out_pages_max, n_tokens=T, page=page, head_dim=D,
                           kv_dtype=kv_dtype)
    L = abi.lib()
    need = L.kvc_compact_pages_workspace(C.byref(a))
    if need == 0:
        raise abi.KvcError(abi.KVC_E_INVALID, "kvc_compact_pages_workspace")
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    abi.check(L.kvc_compact_pages(C.byref(a), ws.data_ptr(), need, _stream(stream)), "kvc_compact_pages")
    out.ws = ws
    return out


class PagedDecoder:
    """Decode attention over per-row page lists (kvc_paged_decode_attn): q [rows][G][128] against the rows' tokens
    in (k_pool, v_pool) [n_pool][page][128]. The workspace is allocated once, for the given page bound."""

    def __init__(self, n_rows: int, group: int, page: int, max_pages: int, kv_dtype: int, device="cuda"):
        self.n_rows, self.group, self.page, self.max_pages, self.kv_dtype = n_rows, group, page, max_pages, kv_dtype
        a = abi.KvcPagedDecodeArgs(q=1 << 12, k_pool=1 << 12, v_pool=1 << 12, page_list=1 << 12, lengths=1 << 12,
                                   out=1 << 12, status=1 << 12, n_rows=n_rows, n_pool_pages=1,
                                   page_stride=max_pages, group=group, page=page, max_pages=max_pages, head_dim=128,
                                   kv_dtype=kv_dtype, reserved=0)
        need = abi.lib().kvc_paged_decode_workspace(C.byref(a))
        if need == 0:
            raise abi.KvcError(abi.KVC_E_INVALID, "kvc_paged_decode_workspace")
        self.ws = torch.empty(need, dtype=torch.uint8, device=device)
        self.status = torch.zeros(1, dtype=torch.int32, device=device)

    def __call__(self, q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor, page_list: torch.Tensor,
                 lengths: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
        n_pool, page, D = k_pool.shape
        assert page == self.page and q.shape == (self.n_rows, self.group, D) and page_list.dim() == 2
        assert page_list.shape[0] == self.n_rows and page_list.shape[1] >= self.max_pages
        out = torch.empty((self.n_rows, self.group, D), dtype=torch.float32, device=q.device) if out is None else out
        a = abi.KvcPagedDecodeArgs(q=q.data_ptr(), k_pool=k_pool.data_ptr(), v_pool=v_pool.data_ptr(),
                                   page_list=page_list.data_ptr(), lengths=lengths.data_ptr(), out=out.data_ptr(),
                                   status=self.status.data_ptr(), n_rows=self.n_rows, n_pool_pages=n_pool,
                                   page_stride=page_list.stride(0), group=self.group, page=page,
                                   max_pages=self.max_pages, head_dim=D, kv_dtype=self.kv_dtype, reserved=0)
        abi.check(abi.lib().kvc_paged_decode_attn(C.byref(a), self.ws.data_ptr(), self.ws.numel(), _stream(stream)),
                  "kvc_paged_decode_attn")
        return out

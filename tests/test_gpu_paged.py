"""GPU parity of the decode over per-row page lists (kvc_paged_decode_attn) against the oracle (needs an MI355X).

Tolerance (fp32 accumulation on the GPU against the fp64 oracle), per (row, head): max|g - r| <= 2e-3 * max|r|.
Covers ragged lengths (0, 1, one short of a page, exact pages, one past, several slices), page sizes 16 and 32,
G = 1, 2, 4, 8, fp16 and bf16, page ids scattered over a pool with unlisted pages, list entries past a row's page
count that must never be read, bad page ids and lengths over the host bound (status bit; the other rows stay
exact), determinism, the full DBTrimKV shape on synthetic page lists with edge rows (sampled rows), and the full
shape on the GPU's own compaction output: score, global top-M and kvc_compact_pages on the device, then the
decode over the fresh pages they leave (sampled rows against the oracle over the kept source rows).
"""
import sys

import numpy as np
import pytest
import torch

from kv_cache_compression_gqa_amd import abi, synth
from kv_cache_compression_gqa_amd.retention import PagedDecoder
from oracle.fp import storage_to_f64
from oracle.paged import paged_gqa_decode

pytestmark = pytest.mark.gpu
RTOL = 2e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _dev(bits, dtype):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()
    return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16)


def _run(inp, group, page, dtype, max_pages=None):
    mp = inp.page_list.shape[1] if max_pages is None else max_pages
    dec = PagedDecoder(len(inp.lengths), group, page, mp, abi.KVC_BF16 if dtype == "bf16" else abi.KVC_F16)
    out = dec(_dev(inp.q, dtype), _dev(inp.k_pool, dtype), _dev(inp.v_pool, dtype),
              torch.from_numpy(inp.page_list).cuda(), torch.from_numpy(inp.lengths).cuda())
    torch.cuda.synchronize()
    return out.cpu().numpy(), int(dec.status.item())


def _check_rows(out, inp, dtype, page, rows=None):
    kp = storage_to_f64(inp.k_pool, dtype)
    vp = storage_to_f64(inp.v_pool, dtype)
    for r in (range(len(inp.lengths)) if rows is None else rows):
        q = storage_to_f64(inp.q[r], dtype)
        ref = paged_gqa_decode(q, kp, vp, inp.page_list[r], int(inp.lengths[r]), page)
        for h in range(ref.shape[0]):
            err = np.abs(out[r, h] - ref[h]).max()
            lim = RTOL * np.abs(ref[h]).max()
            assert err <= lim, f"row {r} (length {inp.lengths[r]}) head {h}: max err {err} > {lim}"


LENGTHS = [0, 1, 15, 16, 17, 31, 33, 255, 256, 257, 700, 1500, 4097]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("group", [1, 2, 4, 8])
@pytest.mark.parametrize("page", [16, 32])
def test_paged_decode_matches_oracle(gpu_lib, dtype, group, page):
    log(f"case: paged decode {dtype} G={group} page={page} lengths {LENGTHS}")
    inp = synth.make_paged(LENGTHS, group, page, seed=40 + group + page, dtype=dtype)
    out, st = _run(inp, group, page, dtype)
    assert st == 0, f"status {st:#x}"
    _check_rows(out, inp, dtype, page)
    assert not out[0].any(), "a row of length 0 must give zeros"


def test_bad_page_ids_and_over_bound_lengths(gpu_lib):
    log("case: bad page ids and lengths over the bound")
    lengths = [40, 300, 64, 500]
    inp = synth.make_paged(lengths, 4, 16, seed=51, max_pages=32)
    ref_inp = synth.make_paged(lengths, 4, 16, seed=51, max_pages=32)
    inp.page_list[1, 3] = 1 << 30      # a bad id in row 1
    inp.page_list[3, 0] = -2           # and in row 3
    out, st = _run(inp, 4, 16, "bf16", max_pages=32)
    assert st & abi.KVC_DEV_BOUND_EXCEEDED
    _check_rows(out, ref_inp, "bf16", 16, rows=[0, 2])   # untouched rows stay exact
    assert np.isfinite(out).all()
    # a length over max_pages * page: the tokens past the bound are ignored
    inp2 = synth.make_paged([600, 100], 4, 16, seed=52, max_pages=40)
    out2, st2 = _run(inp2, 4, 16, "bf16", max_pages=20)
    assert st2 & abi.KVC_DEV_BOUND_EXCEEDED
    cut = synth.make_paged([600, 100], 4, 16, seed=52, max_pages=40)
    cut.lengths[0] = 320
    _check_rows(out2, cut, "bf16", 16)


def test_paged_decode_is_bitwise_reproducible(gpu_lib):
    inp = synth.make_paged([5000, 17, 2048], 8, 16, seed=53)
    a, _ = _run(inp, 8, 16, "bf16")
    b, _ = _run(inp, 8, 16, "bf16")
    assert np.array_equal(a, b)


def test_paged_decode_full_retention_shape(gpu_lib):
    """The DBTrimKV shape after its global budget: 32 layers x 8 KV heads = 256 rows, G = 4, 16-token pages, about
    13107 kept tokens per row (a seeded length mix in [11000, 15000]) plus edge rows (empty, one token, one page,
    one past a page, a row that keeps all 131072 positions); the pools (about 1.8 GB each) are built on the device
    from the seeded table. Every row is checked for finiteness; sampled rows against the oracle."""
    from kv_cache_compression_gqa_amd import configs
    cfg = configs.DBTRIM_128K
    rows, G, page = cfg.layers * cfg.hkv, 4, cfg.page
    rng = np.random.default_rng(77)
    lengths = rng.integers(11000, 15001, size=rows)
    lengths[:5] = [0, 1, page, page + 1, cfg.n_tokens]
    lists = synth.make_large_paged_lists(lengths, G, page, seed=78)
    log(f"case: paged decode full shape, {rows} rows, {int(lengths.sum())} tokens, pool {lists.n_pool} pages")
    kp = synth.device_pool(lists.n_pool, page, 128, lists.k_seed)
    vp = synth.device_pool(lists.n_pool, page, 128, lists.v_seed)
    dec = PagedDecoder(rows, G, page, lists.page_list.shape[1], abi.KVC_BF16)
    out = dec(_dev(lists.q, "bf16"), kp, vp, torch.from_numpy(lists.page_list).cuda(),
              torch.from_numpy(lists.lengths).cuda())
    torch.cuda.synchronize()
    assert int(dec.status.item()) == 0
    out = out.cpu().numpy()
    del kp, vp
    torch.cuda.empty_cache()
    assert np.isfinite(out).all() and not out[0].any()
    for r in [1, 2, 3, 4, 5, 77, 200, rows - 1]:
        n = int(lengths[r])
        pos = np.arange(n)
        ids = lists.page_list[r][pos // page].astype(np.int64) * page + pos % page
        K = storage_to_f64(synth.pool_row_bits(ids, 128, lists.k_seed), "bf16")
        V = storage_to_f64(synth.pool_row_bits(ids, 128, lists.v_seed), "bf16")
        ref = paged_gqa_decode(storage_to_f64(lists.q[r], "bf16"), K.reshape(n, 1, 128), V.reshape(n, 1, 128),
                               np.arange(n), n, 1)
        for h in range(G):
            err = np.abs(out[r, h] - ref[h]).max()
            lim = RTOL * np.abs(ref[h]).max()
            assert err <= lim, f"row {r} (length {n}) head {h}: max err {err} > {lim}"


def test_paged_decode_on_compaction_output(gpu_lib):
    """The whole DBTrimKV path at full size on the device (32 x 8 rows of 131072 positions, M = 10%): log-retention
    scores, the global top-M, kvc_compact_pages into fresh 16-token pages, then the paged decode over those pages.
    Sampled rows are checked against the oracle attending over the row's kept positions, ascending, with K and V
    taken from the source pool rows the page table maps them to."""
    from kv_cache_compression_gqa_amd import configs, retention
    cfg = configs.DBTRIM_128K
    L, H, T, page, D, G = cfg.layers, cfg.hkv, cfg.n_tokens, cfg.page, cfg.head_dim, 4
    rows = L * H
    log(f"case: paged decode on the compaction output, {rows} rows x {T}, M={cfg.keep}")
    beta = torch.from_numpy(synth.make_retention_beta(cfg).reshape(rows, T)).cuda()
    pt_np = synth.make_page_table(cfg).reshape(rows, T // page).astype(np.int32)
    pt = torch.from_numpy(pt_np).cuda()
    seeds = (cfg.seed * 7 + 1, cfg.seed * 7 + 2)
    n_src = rows * (T // page)
    kp_src, vp_src = (synth.device_pool(n_src, page, D, sd, cfg.dtype) for sd in seeds)
    tm = retention.global_topm(retention.retention_scores(beta, cfg.t), cfg.keep)
    comp = retention.compact_pages(tm.keep, pt, kp_src, vp_src, cfg.keep // page + rows + 1, abi.KVC_BF16)
    torch.cuda.synchronize()
    assert int(tm.status.item()) == 0 and int(comp.status.item()) == 0
    keep = tm.keep.cpu().numpy().astype(bool)
    del beta, kp_src, vp_src, tm
    torch.cuda.empty_cache()
    lengths = comp.lengths
    n_pages = comp.n_pages.to(torch.int64)
    max_pages = int(n_pages.max().item())
    col = torch.arange(max_pages, device="cuda", dtype=torch.int64)
    pl = torch.where(col[None, :] < n_pages[:, None], comp.page_offset.to(torch.int64)[:, None] + col[None, :],
                     torch.full_like(col[None, :], -7)).to(torch.int32).contiguous()
    q_bits = synth.to_storage_bits(synth.unit_rng(cfg.seed, 1 << 25).standard_normal((rows, G, D)), "bf16")
    dec = PagedDecoder(rows, G, page, max_pages, abi.KVC_BF16)
    out = dec(_dev(q_bits, "bf16"), comp.k.view(-1, page, D), comp.v.view(-1, page, D), pl, lengths)
    torch.cuda.synchronize()
    assert int(dec.status.item()) == 0
    out = out.cpu().numpy()
    np.testing.assert_array_equal(lengths.cpu().numpy(), keep.sum(axis=1))
    assert np.isfinite(out).all()
    for r in [0, 1, 37, 128, 200, rows - 1]:
        pos = np.nonzero(keep[r])[0]
        n = pos.size
        src = pt_np[r][pos // page].astype(np.int64) * page + pos % page
        K = storage_to_f64(synth.pool_row_bits(src, D, seeds[0], cfg.dtype), "bf16")
        V = storage_to_f64(synth.pool_row_bits(src, D, seeds[1], cfg.dtype), "bf16")
        ref = paged_gqa_decode(storage_to_f64(q_bits[r], "bf16"), K.reshape(n, 1, D), V.reshape(n, 1, D),
                               np.arange(n), n, 1)
        for h in range(G):
            err = np.abs(out[r, h] - ref[h]).max()
            lim = RTOL * np.abs(ref[h]).max()
            assert err <= lim, f"row {r} (length {n}) head {h}: max err {err} > {lim}"
    log("paged decode on the compaction output: sampled rows match")

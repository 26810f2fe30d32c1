"""Seeded synthetic inputs for the compressed-KV decode path.

This module only draws random numbers and lays them out; it holds none of the method's arithmetic, so the CPU
oracle (tests) and the HIP path can both be fed from it.

Structure of a decode workload, per unit u = (layer, batch, kv_head):
  * a unit-level query direction qbar ~ N(0, I_D);
  * prefill keys and values ~ N(0, 1), except
      - ``n_salient`` positions drawn without replacement from [1, len) whose keys are 4 * qbar/|qbar|
        (keys aligned with the queries, logit about +4 above the noise), and
      - position 0 (the attention sink) whose key is 8 * qbar/|qbar|;
  * per decode step: q_h = qbar + eps (eps ~ N(0, I_D)) for each of the G query heads of the group, and one new
    key and value ~ N(0, 1) appended to the cache;
  * everything is cast (round-to-nearest-even) to the K/V storage dtype; queries use the same dtype.

Every unit has its own PCG64 stream, seeded from (workload seed, flat unit id), so any subset of units can be
regenerated on its own.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from .configs import DecodeWorkload, CriticalKVWorkload, RetentionWorkload


def unit_rng(seed: int, unit: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(unit)])))


def to_storage_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float values to the storage dtype (RNE) and return the raw 16-bit patterns."""
    if dtype == "f16":
        return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16)
    raise ValueError(dtype)


def bits_to_f32(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of 16-bit storage patterns to float32 (for building inputs and for display)."""
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float32)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32)
    raise ValueError(dtype)


def sequence_lengths(cfg: DecodeWorkload) -> np.ndarray:
    if cfg.context is not None:
        return np.full(cfg.batch, cfg.context, dtype=np.int64)
    lo, hi = cfg.context_range
    rng = unit_rng(cfg.seed, 1 << 23)
    return rng.integers(lo, hi + 1, size=cfg.batch, dtype=np.int64)


@dataclass
class DecodeInputs:
    """Host arrays for a decode workload (all K/V/q data as 16-bit storage patterns)."""

    cfg: DecodeWorkload
    units: np.ndarray          # [U'] flat unit ids held here
    lengths: np.ndarray        # [U'] prefill length per held unit
    n_windows: np.ndarray      # [U'] routable windows = len // W
    tail0: np.ndarray          # [U'] initial tail length = len % W
    n_windows_max: int
    k_win: np.ndarray          # [U'][NW][W][D] uint16
    v_win: np.ndarray
    k_tail0: np.ndarray        # [U'][W][D] uint16 (first tail0 rows valid)
    v_tail0: np.ndarray
    q: np.ndarray              # [S][U'][G][D] uint16
    k_new: np.ndarray          # [S][U'][D] uint16
    v_new: np.ndarray
    salient: list             # per held unit: sorted salient positions
    qbar: np.ndarray | None = None  # [U'][D] float64 query direction of each held unit


def _unit_decode_draws(cfg: DecodeWorkload, unit: int, length: int, steps: int):
    rng = unit_rng(cfg.seed, unit)
    D = cfg.head_dim
    qbar = rng.standard_normal(D)
    K = rng.standard_normal((length, D))
    V = rng.standard_normal((length, D))
    ns = cfg.salient_count(length)
    sal = np.sort(rng.choice(np.arange(1, length), size=ns, replace=False)) if ns > 0 else np.zeros(0, np.int64)
    direction = qbar / np.linalg.norm(qbar)
    K[sal] = 4.0 * direction
    K[0] = 8.0 * direction
    eps = rng.standard_normal((steps, cfg.group, D))
    q = qbar[None, None, :] + eps
    k_new = rng.standard_normal((steps, D))
    v_new = rng.standard_normal((steps, D))
    return K, V, q, k_new, v_new, sal, qbar


def make_decode(cfg: DecodeWorkload, units=None, steps: int | None = None) -> DecodeInputs:
    """Generate the prefill cache and per-step (q, k, v) for the listed units (default: all)."""
    steps = cfg.steps if steps is None else steps
    all_units = np.arange(cfg.n_units) if units is None else np.asarray(units, dtype=np.int64)
    seq_lens = sequence_lengths(cfg)
    lens = np.array([seq_lens[cfg.unit_coords(int(u))[1]] for u in all_units], dtype=np.int64)
    W, D, G = cfg.window, cfg.head_dim, cfg.group
    nw = lens // W
    NW = max(1, int((seq_lens // W).max()))  # window capacity (at least one slot, even when no window is full)
    Up = len(all_units)
    k_win = np.zeros((Up, NW, W, D), np.uint16)
    v_win = np.zeros((Up, NW, W, D), np.uint16)
    k_t = np.zeros((Up, W, D), np.uint16)
    v_t = np.zeros((Up, W, D), np.uint16)
    q = np.zeros((steps, Up, G, D), np.uint16)
    kn = np.zeros((steps, Up, D), np.uint16)
    vn = np.zeros((steps, Up, D), np.uint16)
    sal_list = []
    qbars = np.zeros((Up, D))
    for j, u in enumerate(all_units):
        L = int(lens[j])
        K, V, qq, k_new, v_new, sal, qbars[j] = _unit_decode_draws(cfg, int(u), L, steps)
        n = int(nw[j]) * W
        kb = to_storage_bits(K, cfg.dtype)
        vb = to_storage_bits(V, cfg.dtype)
        k_win[j, :nw[j]] = kb[:n].reshape(nw[j], W, D)
        v_win[j, :nw[j]] = vb[:n].reshape(nw[j], W, D)
        k_t[j, :L - n] = kb[n:]
        v_t[j, :L - n] = vb[n:]
        q[:, j] = to_storage_bits(qq, cfg.dtype)
        kn[:, j] = to_storage_bits(k_new, cfg.dtype)
        vn[:, j] = to_storage_bits(v_new, cfg.dtype)
        sal_list.append(sal)
    return DecodeInputs(cfg=cfg, units=all_units, lengths=lens, n_windows=nw.astype(np.int64),
                        tail0=(lens - nw * W).astype(np.int64), n_windows_max=NW, k_win=k_win, v_win=v_win,
                        k_tail0=k_t, v_tail0=v_t, q=q, k_new=kn, v_new=vn, salient=sal_list, qbar=qbars)


@dataclass
class SharedLayers:
    """How the units of a many-layer workload start from the held draws of layer 0.

    Unit u = (layer l, sequence b, KV head g) starts from held unit j = unit_map[u] = (0, b, g), with:
      * its prefill windows rotated by rot[u] = (37 * l) mod n_windows: window w of unit u holds held window
        (w + rot[u]) mod n_windows (an index permutation: the layers of one (b, g) hold the same key and value rows
        at different window positions, so a read of another layer's unit returns other data);
      * the held prefill tail as it is;
      * per-step inputs of its own: q_h = qbar_j + eps with eps ~ N(0, I_D), and a new key and value ~ N(0, 1) per
        step, drawn from unit u's own stream (layer 0 keeps the held draws).
    """

    unit_map: np.ndarray  # [U] held unit of each unit
    rot: np.ndarray       # [U] window rotation
    q: np.ndarray         # [S][U][G][D] storage bits
    k_new: np.ndarray     # [S][U][D] storage bits
    v_new: np.ndarray

    def window_order(self, inp: DecodeInputs, u: int) -> np.ndarray:
        """Held window ids of unit u's windows 0 .. n_windows - 1."""
        nw = int(inp.n_windows[int(self.unit_map[u])])
        return (np.arange(nw) + int(self.rot[u])) % max(nw, 1)


def make_decode_shared_layers(cfg: DecodeWorkload, steps: int | None = None):
    """Held inputs for the units of layer 0 (one seeded draw per (sequence, KV head), each at its sequence's
    length) and the ``SharedLayers`` plan that starts every unit (layer l, b, g) from held unit (0, b, g) with its
    windows rotated per layer and per-step inputs of its own. Every unit then holds its own memory, state and
    data order; drawing every layer's whole prefill on the host would take minutes at 32 layers x batch 16."""
    steps = cfg.steps if steps is None else steps
    base = np.array([cfg.unit_index(0, b, g) for b in range(cfg.batch) for g in range(cfg.hkv)], dtype=np.int64)
    inp = make_decode(cfg, units=base, steps=steps)
    U, G, D = cfg.n_units, cfg.group, cfg.head_dim
    coords = [cfg.unit_coords(u) for u in range(U)]
    umap = np.array([b * cfg.hkv + g for (_, b, g) in coords], dtype=np.int64)
    layer = np.array([l for (l, _, _) in coords], dtype=np.int64)
    nw = inp.n_windows[umap]
    rot = np.where(nw > 0, (37 * layer) % np.maximum(nw, 1), 0).astype(np.int64)
    q = np.zeros((steps, U, G, D))
    kn = np.zeros((steps, U, D))
    vn = np.zeros((steps, U, D))
    held = layer == 0
    for u in np.nonzero(~held)[0]:
        rng = unit_rng(cfg.seed, int(u))
        q[:, u] = inp.qbar[umap[u]][None, None, :] + rng.standard_normal((steps, G, D))
        kn[:, u] = rng.standard_normal((steps, D))
        vn[:, u] = rng.standard_normal((steps, D))
    qb = to_storage_bits(q, cfg.dtype)
    kb = to_storage_bits(kn, cfg.dtype)
    vb = to_storage_bits(vn, cfg.dtype)
    h = np.nonzero(held)[0]
    qb[:, h] = inp.q[:, umap[h]]
    kb[:, h] = inp.k_new[:, umap[h]]
    vb[:, h] = inp.v_new[:, umap[h]]
    return inp, SharedLayers(unit_map=umap, rot=rot, q=qb, k_new=kb, v_new=vb)


# ----------------------------------------------------------------------------------------------------------
# CriticalKV prefill-selection inputs


@dataclass
class CriticalKVInputs:
    cfg: CriticalKVWorkload
    q_obs: np.ndarray   # [Hq][n_obs][D] uint16 (queries at positions n - n_obs + j)
    k: np.ndarray       # [Hkv][n][D] uint16
    v: np.ndarray       # [Hkv][n][D] uint16
    w_o: np.ndarray     # [Hq*D][d_model] uint16, row index = h*D + d (input feature), column = output feature
    salient: list


def make_criticalkv(cfg: CriticalKVWorkload, n_keys: int | None = None, d_model: int | None = None,
                    n_salient: int | None = None) -> CriticalKVInputs:
    """Inputs for the observation-window selection. ``n_keys``/``d_model``/``n_salient`` shrink it for tests."""
    n = cfg.n_keys if n_keys is None else n_keys
    dm = cfg.d_model if d_model is None else d_model
    ns = cfg.n_salient if n_salient is None else n_salient
    D, G, T = cfg.head_dim, cfg.group, cfg.n_obs
    q = np.zeros((cfg.hq, T, D), np.uint16)
    k = np.zeros((cfg.hkv, n, D), np.uint16)
    v = np.zeros((cfg.hkv, n, D), np.uint16)
    sal_list = []
    for g in range(cfg.hkv):
        rng = unit_rng(cfg.seed, g)
        qbar = rng.standard_normal(D)
        K = rng.standard_normal((n, D))
        V = rng.standard_normal((n, D))
        hi = max(2, n - T - 1)
        sal = np.sort(rng.choice(np.arange(1, hi), size=min(ns, hi - 1), replace=False))
        direction = qbar / np.linalg.norm(qbar)
        K[sal] = 4.0 * direction
        K[0] = 8.0 * direction
        eps = rng.standard_normal((G, T, D))
        q[g * G:(g + 1) * G] = to_storage_bits(qbar[None, None, :] + eps, cfg.dtype)
        k[g] = to_storage_bits(K, cfg.dtype)
        v[g] = to_storage_bits(V, cfg.dtype)
        sal_list.append(sal)
    rng = unit_rng(cfg.seed, 1 << 20)
    w = rng.standard_normal((cfg.hq * D, dm)) / 64.0
    return CriticalKVInputs(cfg=cfg, q_obs=q, k=k, v=v, w_o=to_storage_bits(w, cfg.dtype), salient=sal_list)


# ----------------------------------------------------------------------------------------------------------
# DBTrimKV global-budget inputs


def make_retention_beta(cfg: RetentionWorkload, layers: int | None = None, n_tokens: int | None = None):
    """Per-entry retention beta ~ Beta(a, b), clipped to [2^-24, 1 - 2^-24], float32, shape [L][Hkv][T]."""
    L = cfg.layers if layers is None else layers
    T = cfg.n_tokens if n_tokens is None else n_tokens
    out = np.empty((L, cfg.hkv, T), np.float32)
    for l in range(L):
        rng = unit_rng(cfg.seed, l)
        b = rng.beta(cfg.beta_a, cfg.beta_b, size=(cfg.hkv, T))
        out[l] = np.clip(b, 2.0 ** -24, 1.0 - 2.0 ** -24).astype(np.float32)
    return out


def make_page_table(cfg: RetentionWorkload, layers: int | None = None, n_tokens: int | None = None):
    """Source page table [L][Hkv][T/page] int32: a seeded permutation of all page ids."""
    L = cfg.layers if layers is None else layers
    T = cfg.n_tokens if n_tokens is None else n_tokens
    n_pages = L * cfg.hkv * (T // cfg.page)
    rng = unit_rng(cfg.seed, 1 << 21)
    return rng.permutation(n_pages).astype(np.int32).reshape(L, cfg.hkv, T // cfg.page)


def pool_row_index(row_ids, pool_rows: int = 1 << 16):
    """Table row of pool row r: (r * 40503 + 17 + (r >> 16) * 7919) mod pool_rows (numpy or torch int64). The
    second term shifts every block of 65536 rows by a different odd offset, so rows repeat only every 2^32."""
    return (row_ids * 40503 + 17 + (row_ids >> 16) * 7919) % pool_rows


def pool_row_bits(row_ids: np.ndarray, head_dim: int, seed: int, dtype: str = "bf16",
                  pool_rows: int = 1 << 16) -> np.ndarray:
    """K/V pool rows for the paged cache: row r (global row id = page*page_size + slot) takes table row
    ``pool_row_index(r)`` of a seeded N(0,1) table, so huge pools need only a small table."""
    table = pool_table_bits(head_dim, seed, dtype, pool_rows)
    return table[pool_row_index(np.asarray(row_ids).astype(np.int64), pool_rows)]


_POOL_CACHE: dict = {}


def pool_table_bits(head_dim: int, seed: int, dtype: str = "bf16", pool_rows: int = 1 << 16) -> np.ndarray:
    key = (head_dim, seed, dtype, pool_rows)
    if key not in _POOL_CACHE:
        rng = unit_rng(seed, 1 << 22)
        _POOL_CACHE[key] = to_storage_bits(rng.standard_normal((pool_rows, head_dim)), dtype)
    return _POOL_CACHE[key]


# ----------------------------------------------------------------------------------------------------------
# Inputs of the decode over per-row page lists


@dataclass
class PagedInputs:
    q: np.ndarray          # [rows][G][D] storage bits
    k_pool: np.ndarray     # [n_pool][page][D] storage bits
    v_pool: np.ndarray
    page_list: np.ndarray  # [rows][max_pages] int32; entries past a row's page count are -7 (never read)
    lengths: np.ndarray    # [rows] int32


def make_paged(lengths, group: int, page: int, seed: int, dtype: str = "bf16", spare_pages: int = 3,
               head_dim: int = 128, max_pages: int | None = None) -> PagedInputs:
    """Rows of the given lengths, their pages at distinct random ids of a pool with ``spare_pages`` unlisted
    pages. q ~ N(0, I); keys and values ~ N(0, 1), except that every row has four keys along its mean query
    direction (logit about 6 for that mean), so the softmax has both flat and peaked parts."""
    lengths = np.asarray(lengths, np.int64)
    rows = lengths.size
    n_pages = (lengths + page - 1) // page
    mp = max(1, int(n_pages.max()) if rows else 1) if max_pages is None else max_pages
    n_pool = int(n_pages.sum()) + spare_pages
    rng = np.random.default_rng(seed)
    ids = rng.permutation(n_pool).astype(np.int32)
    page_list = np.full((rows, mp), -7, np.int32)
    q = rng.standard_normal((rows, group, head_dim))
    K = rng.standard_normal((n_pool, page, head_dim))
    V = rng.standard_normal((n_pool, page, head_dim))
    off = 0
    for r in range(rows):
        page_list[r, :n_pages[r]] = ids[off:off + n_pages[r]]
        off += int(n_pages[r])
        if lengths[r] > 0:
            qm = q[r].mean(0)
            key = 6.0 * np.sqrt(head_dim) * qm / (np.linalg.norm(qm) ** 2 + 1e-12)  # logit about 6 for the mean query
            for i in rng.choice(int(lengths[r]), size=min(4, int(lengths[r])), replace=False):
                K[page_list[r, i // page], i % page] = key
    return PagedInputs(q=to_storage_bits(q, dtype), k_pool=to_storage_bits(K, dtype),
                       v_pool=to_storage_bits(V, dtype), page_list=page_list, lengths=lengths.astype(np.int32))


@dataclass
class LargePagedLists:
    q: np.ndarray          # [rows][G][D] storage bits, q ~ N(0, I)
    page_list: np.ndarray  # [rows][max_pages] int32 (-7 past a row's page count)
    lengths: np.ndarray    # [rows] int32
    n_pool: int            # pool pages; pool row r = page * page_size + slot takes pool_row_bits([r], ...)
    k_seed: int
    v_seed: int


def make_large_paged_lists(lengths, group: int, page: int, seed: int, dtype: str = "bf16", spare_pages: int = 5,
                           head_dim: int = 128) -> LargePagedLists:
    """Per-row page lists for a pool too large to draw on the host: the rows' pages are distinct ids of a seeded
    permutation of the pool; the pool's K and V rows are defined by ``pool_row_bits`` (seeds ``k_seed`` and
    ``v_seed``), so a device gather of ``pool_table_bits`` builds the pools and the host regenerates any row."""
    lengths = np.asarray(lengths, np.int64)
    n_pages = (lengths + page - 1) // page
    n_pool = int(n_pages.sum()) + spare_pages
    rng = unit_rng(seed, 1 << 24)
    ids = rng.permutation(n_pool).astype(np.int32)
    page_list = np.full((lengths.size, max(1, int(n_pages.max()))), -7, np.int32)
    off = np.concatenate([[0], np.cumsum(n_pages)])
    for r in range(lengths.size):
        page_list[r, :n_pages[r]] = ids[off[r]:off[r + 1]]
    q = to_storage_bits(rng.standard_normal((lengths.size, group, head_dim)), dtype)
    return LargePagedLists(q=q, page_list=page_list, lengths=lengths.astype(np.int32), n_pool=n_pool,
                           k_seed=seed * 7 + 3, v_seed=seed * 7 + 4)


def device_pool(n_pages: int, page: int, head_dim: int, seed: int, dtype: str = "bf16", device="cuda"):
    """The pool [n_pages][page][head_dim] (storage dtype) whose row r is pool_row_bits([r], ...): a device gather
    of the seeded table (an index permutation only)."""
    tab = torch.from_numpy(pool_table_bits(head_dim, seed, dtype).view(np.int16)).to(device)
    idx = pool_row_index(torch.arange(n_pages * page, device=device, dtype=torch.int64), tab.shape[0])
    out = tab[idx].view(torch.bfloat16 if dtype == "bf16" else torch.float16).view(n_pages, page, head_dim)
    del idx
    return out

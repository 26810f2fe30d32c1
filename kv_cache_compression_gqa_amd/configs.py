"""Workload shapes for the compressed-KV GQA decode path.

Five workloads, named by what they are. Sizes, budgets and cadences are the ones the source pages' long-context
settings call for (QEvict: windowed three-tier routing with INT2 recoverable tier; DBTrimKV: one global top-M
with per-head paged lists; CriticalKV: two-stage selection with alpha = 0.5). Nothing here computes anything
of the method; it only states shapes.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional, Tuple

HEAD_DIM = 128
WINDOW = 32
INT2_GROUP = 32


@dataclass(frozen=True)
class DecodeWorkload:
    """Windowed three-tier decode (QEvict page, 'Metodologia' and 'Mecanismos Principais')."""

    name: str
    seed: int
    layers: int
    batch: int
    hq: int
    hkv: int
    dtype: str  # "f16" | "bf16"
    context: Optional[int] = None            # fixed per-sequence length
    context_range: Optional[Tuple[int, int]] = None  # inclusive uniform range per sequence
    n_salient: Optional[int] = None          # literal count per unit
    salient_frac: Optional[float] = None     # floor(frac * len) per unit
    budget_full: Optional[int] = None        # literal window counts per unit
    budget_int2: Optional[int] = None
    frac_full: Optional[float] = None        # floor(frac * n_windows) per unit
    frac_int2: Optional[float] = None
    steps: int = 8
    route_every: int = 4
    head_dim: int = HEAD_DIM
    window: int = WINDOW

    @property
    def group(self) -> int:
        return self.hq // self.hkv

    @property
    def n_units(self) -> int:
        return self.layers * self.batch * self.hkv

    def seq_len(self, lengths=None, b: int = 0) -> int:
        if self.context is not None:
            return self.context
        assert lengths is not None
        return int(lengths[b])

    def unit_index(self, layer: int, b: int, g: int) -> int:
        """Flat unit id; units of one sequence and layer are contiguous."""
        return (layer * self.batch + b) * self.hkv + g

    def unit_coords(self, u: int):
        g = u % self.hkv
        lb = u // self.hkv
        return lb // self.batch, lb % self.batch, g

    def salient_count(self, length: int) -> int:
        if self.n_salient is not None:
            return self.n_salient
        return int(math.floor(self.salient_frac * length))

    def budgets(self, n_windows: int) -> Tuple[int, int]:
        if self.budget_full is not None:
            return self.budget_full, self.budget_int2
        return int(math.floor(self.frac_full * n_windows)), int(math.floor(self.frac_int2 * n_windows))


@dataclass(frozen=True)
class CriticalKVWorkload:
    """Two-stage perturbation-constrained selection (CriticalKV page, 'Algoritmo', Algorithm 1)."""

    name: str
    seed: int
    n_keys: int
    hq: int
    hkv: int
    n_obs: int
    budget: int
    alpha: float
    n_salient: int
    dtype: str = "bf16"
    head_dim: int = HEAD_DIM

    @property
    def group(self) -> int:
        return self.hq // self.hkv

    @property
    def d_model(self) -> int:
        return self.hq * self.head_dim


@dataclass(frozen=True)
class RetentionWorkload:
    """Global retention top-M over all layers and heads (DBTrimKV page, 'Metodologia' sections 2-4)."""

    name: str
    seed: int
    layers: int
    hkv: int
    n_tokens: int
    page: int
    keep_frac: float
    beta_a: float = 8.0
    beta_b: float = 2.0
    head_dim: int = HEAD_DIM
    dtype: str = "bf16"

    @property
    def t(self) -> int:
        return self.n_tokens

    @property
    def n_entries(self) -> int:
        return self.layers * self.hkv * self.n_tokens

    @property
    def keep(self) -> int:
        return int(math.floor(self.keep_frac * self.n_entries))

    @property
    def pages_per_head(self) -> int:
        return self.n_tokens // self.page


TINY = DecodeWorkload(
    name="tiny_gqa4_ctx1k_f16", seed=1, layers=1, batch=1, hq=8, hkv=2, dtype="f16", context=1024,
    n_salient=16, budget_full=8, budget_int2=8, steps=8, route_every=4)

LLAMA3_8B_LAYER_32K = DecodeWorkload(
    name="llama3_8b_layer_ctx32k_bf16", seed=2, layers=1, batch=1, hq=32, hkv=8, dtype="bf16", context=32768,
    salient_frac=0.01, frac_full=0.2, frac_int2=0.3, steps=64, route_every=16)

BATCHED_32L_B16 = DecodeWorkload(
    name="batched_32l_b16_ctx4k_8k_bf16", seed=3, layers=32, batch=16, hq=32, hkv=8, dtype="bf16",
    context_range=(4096, 8192), salient_frac=0.01, frac_full=0.25, frac_int2=0.25, steps=8, route_every=1)

CRITICALKV_64K = CriticalKVWorkload(
    name="criticalkv_prefill_64k_bf16", seed=4, n_keys=65536, hq=32, hkv=8, n_obs=32, budget=2048, alpha=0.5,
    n_salient=655)

DBTRIM_128K = RetentionWorkload(
    name="dbtrim_global_32l_8h_128k", seed=5, layers=32, hkv=8, n_tokens=131072, page=16, keep_frac=0.1)

DECODE_WORKLOADS = {w.name: w for w in (TINY, LLAMA3_8B_LAYER_32K, BATCHED_32L_B16)}

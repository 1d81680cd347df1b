"""Workload descriptions for block-sparse prefill attention.

Each workload is a single attention layer with a causal prefill over a paged
KV cache.  The shapes follow the two backbones the CoSA paper evaluates
(CoSA (paperpeel), §5.1 "Baselines and models": Llama-3.1-8B-Instruct and
Qwen3-8B, both 32 query heads / 8 KV heads, head_dim 128) at the context
lengths it reports speed for (§5.3 "Attention speedup", up to 128K).

The planted structure (attention sink, local band, vertical stripes, outlier
key channels) stands in for the sink / local / vertical-stripe patterns that
the proxies discussed in the paper target (CoSA (paperpeel), App. B.1).  No
dataset or trained weight is involved: every value is drawn from a seeded
generator in :mod:`cosa_inputs.generate`.

This module holds descriptions only; it contains none of the attention or
selection arithmetic.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Dict, Optional, Tuple


@dataclass(frozen=True)
class HeadPattern:
    """Planted structure for one KV head (shared by its query-head group)."""

    sink: bool = True          # key block 0 gets sink_strength * u_g
    band: int = 0              # local band width in KV blocks (0 = none)
    stripes: int = 0           # number of vertical-stripe key blocks
    strength: float = 3.0      # s: stripe / band strength
    sink_strength: Optional[float] = None  # default 2 * strength
    q_dir: bool = True         # add u_g to every query of the group

    def sink_value(self) -> float:
        return 2.0 * self.strength if self.sink_strength is None else self.sink_strength


@dataclass(frozen=True)
class Workload:
    name: str
    seqlens: Tuple[int, ...]
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    q_block: int
    page_size: int
    budget: float
    tau: float
    seed: int
    # value precision the workload is specified in ("fp32" keeps raw fp32
    # values for CPU self-tests; the GPU always consumes bf16-rounded copies)
    precision: str = "bf16"
    shuffled_pages: bool = True
    spare_pages: int = 64
    pattern: HeadPattern = field(default_factory=HeadPattern)
    # optional per-KV-head pattern mix: tuple of (fraction, HeadPattern)
    pattern_mix: Optional[Tuple[Tuple[float, HeadPattern], ...]] = None
    outlier_channels: int = 0
    outlier_scale: float = 10.0
    # extra query/key pushes used only by test variants
    q_dir_gain: float = 1.0
    # logical key block of the sparse path (None: one page)
    kv_block: Optional[int] = None
    budgets_sweep: Tuple[float, ...] = ()
    taus_sweep: Tuple[float, ...] = ()

    @property
    def batch(self) -> int:
        return len(self.seqlens)

    @property
    def total_tokens(self) -> int:
        return int(sum(self.seqlens))

    @property
    def max_seqlen(self) -> int:
        return int(max(self.seqlens)) if self.seqlens else 0

    @property
    def block(self) -> int:
        """Tokens per logical key block."""
        return self.page_size if self.kv_block is None else self.kv_block

    @property
    def softmax_scale(self) -> float:
        return 1.0 / float(self.head_dim) ** 0.5

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


TINY = Workload(
    name="tiny",
    seqlens=(2048,), num_q_heads=2, num_kv_heads=2, head_dim=64,
    q_block=64, page_size=64, budget=0.5, tau=8.0, seed=1,
    precision="fp32", shuffled_pages=False, spare_pages=0,
    pattern=HeadPattern(sink=True, band=2, stripes=3, strength=4.0),
)

LLAMA_32K = Workload(
    name="llama32k",
    seqlens=(32768,), num_q_heads=32, num_kv_heads=8, head_dim=128,
    q_block=128, page_size=64, budget=0.2, tau=8.0, seed=2,
    pattern=HeadPattern(sink=True, band=2, stripes=3, strength=3.0),
)

LLAMA_128K = Workload(
    name="llama128k",
    seqlens=(131072,), num_q_heads=32, num_kv_heads=8, head_dim=128,
    q_block=128, page_size=64, budget=0.1, tau=8.0, seed=3,
    pattern=HeadPattern(sink=True, band=4, stripes=8, strength=3.0),
    budgets_sweep=(0.3, 0.2, 0.1, 0.05), taus_sweep=(6.0, 8.0, 12.0),
)

QWEN_128K = Workload(
    name="qwen128k",
    seqlens=(131072,), num_q_heads=32, num_kv_heads=8, head_dim=128,
    q_block=128, page_size=64, budget=0.1, tau=8.0, seed=4,
    pattern_mix=(
        (0.50, HeadPattern(sink=True, band=0, stripes=16, strength=3.0)),
        (0.25, HeadPattern(sink=False, band=8, stripes=0, strength=3.0, q_dir=False)),
        (0.25, HeadPattern(sink=False, band=0, stripes=0, strength=3.0, q_dir=False)),
    ),
)

STRESS = Workload(
    name="stress",
    seqlens=(16384, 49152, 98304, 131072), num_q_heads=32, num_kv_heads=8,
    head_dim=128, q_block=128, page_size=64, budget=0.1, tau=8.0, seed=5,
    pattern=HeadPattern(sink=True, band=2, stripes=3, strength=3.0),
    outlier_channels=5, outlier_scale=10.0,
)

# Remapping ablation: no sink, a strong local band (about 12.7 nats above the
# noise at D 128) and no query push, so the row maxima sit on the last blocks
# of each tile's causal range.  Visiting the HRM blocks first establishes the
# running max at once; ascending order reaches it only at the end.
REMAP_32K = LLAMA_32K.with_(
    name="remap32k", seed=6, budget=0.3, tau=6.0,
    pattern=HeadPattern(sink=False, band=4, stripes=0, strength=12.0, q_dir=False),
    budgets_sweep=(1.0, 0.3), taus_sweep=(2.0, 4.0, 6.0, 8.0),
)

# Band-only structure at 128K with the Llama shape, for the in-kernel skip.
# With the sink and the weak stripes of llama128k no whole 128-row tile ever
# falls tau below its running max, so the skip never fires there.  Here the
# row maxima sit on the band blocks (about s^2 / sqrt(D) = 22.6 nats above the
# noise) that the HRM group visits first, and the skip decides a large part
# of the rest of each tile's walk: up to 205 visited blocks per tile at the
# 10% budget, 615 at 30%.  (A band of s = 12 skips nothing at tau 8: the
# random band vectors of different blocks leak about +-2.5 nats into every
# logit, so some row of every tile stays within 8 nats of its max.)
REMAP_128K = LLAMA_128K.with_(
    name="remap128k", seed=7, budget=0.1, tau=8.0,
    pattern=HeadPattern(sink=False, band=4, stripes=0, strength=16.0, q_dir=False),
    budgets_sweep=(0.3, 0.1), taus_sweep=(2.0, 4.0, 6.0, 8.0),
)

# The llama128k layer over logical key blocks of 128 keys (two 64-token pages
# each): half the candidate blocks for the proxy, the same budget fraction.
LLAMA_128K_KV128 = LLAMA_128K.with_(name="llama128k_kv128", kv_block=128)

# Test-only variant of the tiny case with a strong sink so that the in-kernel
# skip actually fires (sink logit around 16 nats); not a benchmark workload.
TINY_SKIP = TINY.with_(
    name="tiny_skip", q_dir_gain=8.0,
    pattern=HeadPattern(sink=True, band=2, stripes=3, strength=4.0,
                        sink_strength=2.0 * 8.0),  # 2/scale at D=64
)

WORKLOADS: Dict[str, Workload] = {
    w.name: w for w in (TINY, LLAMA_32K, LLAMA_128K, QWEN_128K, STRESS, REMAP_32K, REMAP_128K,
                         LLAMA_128K_KV128, TINY_SKIP)
}


def get(name: str) -> Workload:
    try:
        return WORKLOADS[name]
    except KeyError as e:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(WORKLOADS)}") from e

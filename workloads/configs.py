"""The five synthetic prefill workloads and their selection settings.

Each workload names its shapes (sequence length, query/key-value heads, head
dimension, block size), the input precision, the selection unit (one list per
query head, or one list per GQA group), the selection rule's parameters and the
structure planted in the inputs.  ``scaled()`` derives a smaller workload with
the same structure for tests the CPU oracle must finish in seconds.

Sources for the five workloads (the pages' own workloads these stand in for):
  tiny        -- the top-k selector over key blocks ("Uncertainty-gated selection
                 for block-sparse attention", technical summary, Methodology
                 steps 1-2), at a size a CPU checks in seconds.
  gqa32k      -- mean-pooled centroid scoring with top-k (same page, step 1, the
                 SSA-style mean-pooling backbone) on a Llama-style GQA layer.
  gated64k    -- the same selector with the uncertainty gate of the lay summary
                 ("The Solution": a tiny top-1/top-2 gap doubles the budget).
  dual128k    -- RBS-Attention's base (centroid) branch and radius rescue branch
                 with masks unioned (RBS-Attention article, third paragraph).
  msa1m       -- MiniMax Sparse Attention's index branch per GQA group feeding
                 the main branch (MSA article, "What is MSA and how does it
                 work"), in FP8 as RBS-Attention measures.
"""

from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field


@dataclass(frozen=True)
class WorkloadConfig:
    name: str
    index: int  # seed root: sub-seeds are index*1000 + stream
    seq_len: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    dtype: str  # "bf16" or "fp8"
    granularity: str  # "qhead" (one list per query head) or "group" (one per GQA group)
    # selection
    top_k: int = 0
    force_sink: bool = False
    gate: str = "none"  # "none", "top12_gap" or "sigma_cut"
    gate_threshold: float = 0.05
    gate_factor: int = 2
    score_temperature: float = 1.0
    mass_threshold: float = 0.0  # 0 = base mass branch off
    rescue_fraction: float = 0.0  # 0 = rescue branch off
    backbone: str = "mean_pool"  # "mean_pool" (pooled-query centroid scores) or "quest"
    # planted structure
    structure: str = "needles"  # "needles", "pairs", "mixture"
    low_rank: int = 0
    low_rank_scale: float = 2.0
    num_needles: int = 0
    needle_range: tuple = (1, -3)  # needles drawn from blocks [lo, nb + hi]
    pairs_per_kv_head: int = 16
    planted_query_fraction: float = 0.30
    pair_magnitude: float = 8.0
    pair_query_gain: float = 8.0
    decoy_sigma: float = 0.01
    tight_sigma: float = 0.1
    wide_sigma: float = 1.5
    extra: dict = field(default_factory=dict)

    @property
    def num_blocks(self) -> int:
        return -(-self.seq_len // self.block_size)

    @property
    def group_size(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def num_units(self) -> int:
        return self.num_q_heads if self.granularity == "qhead" else self.num_kv_heads


CONFIGS = [
    WorkloadConfig(
        name="tiny", index=1, seq_len=1024, num_q_heads=1, num_kv_heads=1, head_dim=64,
        block_size=64, dtype="bf16", granularity="qhead", top_k=4, force_sink=True,
        structure="needles", low_rank=0, num_needles=2, needle_range=(1, -2),
    ),
    WorkloadConfig(
        name="gqa32k", index=2, seq_len=32768, num_q_heads=32, num_kv_heads=8, head_dim=128,
        block_size=128, dtype="bf16", granularity="qhead", top_k=32, force_sink=True,
        structure="needles", low_rank=8, num_needles=16,
    ),
    WorkloadConfig(
        name="gated64k", index=3, seq_len=65536, num_q_heads=32, num_kv_heads=8, head_dim=128,
        block_size=128, dtype="bf16", granularity="qhead", top_k=32, force_sink=True,
        gate="top12_gap", gate_threshold=0.05, gate_factor=2, score_temperature=1.0,
        structure="pairs", low_rank=8,
    ),
    WorkloadConfig(
        name="dual128k", index=4, seq_len=131072, num_q_heads=32, num_kv_heads=4, head_dim=128,
        block_size=128, dtype="bf16", granularity="qhead", top_k=0, force_sink=False,
        score_temperature=1.0, mass_threshold=0.90, rescue_fraction=0.05,
        structure="mixture", low_rank=8,
    ),
    WorkloadConfig(
        name="msa1m", index=5, seq_len=1048576, num_q_heads=64, num_kv_heads=8, head_dim=128,
        block_size=128, dtype="fp8", granularity="group", top_k=64, force_sink=False,
        structure="needles", low_rank=16, num_needles=64,
    ),
]


# Beyond the five: the 128K dual-branch workload with E4M3 inputs (per-(head,
# block) scales), the precision RBS-Attention reports its 128K results in
# (RBS-Attention article, fourth paragraph).  Same seeds and structure as
# dual128k, quantised.
#
# The 64K gated workload under the page's own gate instead of the lay summary's:
# per (tile, head) the normalised cut margin sigma, its mean over heads per tile,
# and expansion to rho*k of the tiles in the lowest q = 0.30 of the layer's
# distribution ("Uncertainty-gated selection for block-sparse attention",
# technical summary, Methodology steps 3-5; q matches the fraction of query
# blocks the generator plants near-ties in).  Same seeds and inputs as gated64k.
#
# The same router on the Quest backbone, the pairing behind the page's LongBench-v2
# result: K-min/K-max per key block, per-row upper bounds, a tile's score the
# maximum over its rows (same page, Methodology steps 1-2 and Results).
_BASE = {c.name: c for c in CONFIGS}
EXTRA_CONFIGS = [
    dataclasses.replace(_BASE["dual128k"], name="dual128k_fp8", dtype="fp8"),
    dataclasses.replace(_BASE["gated64k"], name="sigma64k", gate="sigma_cut", gate_threshold=0.30),
    dataclasses.replace(_BASE["gated64k"], name="quest64k", gate="sigma_cut", gate_threshold=0.30,
                        backbone="quest"),
]


def config_by_name(name: str) -> WorkloadConfig:
    for c in CONFIGS + EXTRA_CONFIGS:
        if c.name == name:
            return c
    raise KeyError(name)


def scaled(cfg: WorkloadConfig, seq_len: int, num_q_heads: int | None = None,
           num_kv_heads: int | None = None, **over) -> WorkloadConfig:
    """Same workload structure at a smaller size (for CPU-checkable tests).

    ``seq_len`` need not be a multiple of the block size: the last block is
    then ragged.  Needle and pair counts shrink with the block count.
    """
    hq = num_q_heads if num_q_heads is not None else cfg.num_q_heads
    hkv = num_kv_heads if num_kv_heads is not None else cfg.num_kv_heads
    name = over.pop("name", f"{cfg.name}@{seq_len}")
    nb = -(-seq_len // over.get("block_size", cfg.block_size))
    kw = dict(seq_len=seq_len, num_q_heads=hq, num_kv_heads=hkv)
    if cfg.num_needles:
        kw["num_needles"] = max(1, min(cfg.num_needles, nb // 4))
    if cfg.structure == "pairs":
        kw["pairs_per_kv_head"] = max(1, min(cfg.pairs_per_kv_head, nb // 8))
    kw.update(over)
    return dataclasses.replace(cfg, name=name, **kw)

"""The five decode workloads, with every choice the pages leave open made explicit.

Block sizes are in tokens (the page "大模型推理KV Cache内存管理与PagedAttention分页显存实战"
gives 16 as the default and 32 for sequences of 8K tokens and more).  The cache
layout is [num_blocks, block_size, num_kv_heads, head_dim] (page
"vLLM推理引擎架构：PagedAttention机制与高吞吐推理", section 2.2, with the head count
read as the number of KV heads).
"""

from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass
from typing import Optional, Tuple

# storage dtype names shared by the generator, the binding and the oracle wrapper
KV_DTYPES = ("f32", "f16", "bf16", "fp8")
Q_DTYPES = ("f32", "f16", "bf16")


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    seed: int
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int  # physical pool size
    max_blocks_per_seq: int  # block-table width W
    kv_dtype: str
    q_dtype: str
    # context-length distribution
    ctx_kind: str  # "fixed" | "uniform" | "lognormal"
    ctx_fixed: Tuple[int, ...] = ()
    ctx_lo: int = 1
    ctx_hi: int = 1
    ctx_median: float = 0.0
    ctx_sigma: float = 0.0
    # physical placement
    allocator: str = "shuffled"  # "permutation" | "shuffled" | "prefix" | "churn"
    share_group: int = 1  # sequences per prefix-sharing group
    share_prefix_blocks: int = 0  # blocks of the shared prefix
    churn_band: Tuple[float, float] = (0.70, 0.90)
    partition_size: int = 0  # tokens per split-context partition, 0 = library choice
    scale: Optional[float] = None  # softmax scale, default 1/sqrt(head_dim)
    # fp8 caches: "tensor" = one scale per K / V tensor, "head" = one per kv head,
    # "block" = one per (physical block, kv head)
    fp8_scales: str = "tensor"
    # standard deviation of kv head h's K and V values, geometric from the first
    # to the second number over the heads (heads of different magnitude)
    head_std: Tuple[float, float] = (1.0, 1.0)

    @property
    def group_size(self) -> int:
        return self.num_heads // self.num_kv_heads

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.head_dim)

    def describe(self) -> dict:
        d = dataclasses.asdict(self)
        d["softmax_scale"] = self.softmax_scale
        return d


CONFIGS = {
    # Tiny MHA fp32 case with a 4-token cache write; 64 physical blocks handed
    # out by a seeded permutation.
    "tiny": DecodeConfig(
        name="tiny", seed=1, num_seqs=4, num_heads=4, num_kv_heads=4, head_dim=64,
        block_size=16, num_blocks=64, max_blocks_per_seq=4, kv_dtype="f32", q_dtype="f32",
        ctx_kind="fixed", ctx_fixed=(1, 17, 33, 64), allocator="permutation",
        scale=1.0 / 8.0,
    ),
    # LLaMA-7B-shaped single layer: 32 heads of 128, fp16, block 16, U[1, 2048].
    "llama7b": DecodeConfig(
        name="llama7b", seed=2, num_seqs=32, num_heads=32, num_kv_heads=32, head_dim=128,
        block_size=16, num_blocks=5000, max_blocks_per_seq=128, kv_dtype="f16", q_dtype="f16",
        ctx_kind="uniform", ctx_lo=1, ctx_hi=2048, allocator="shuffled",
    ),
    # LLaMA-13B-shaped with prefix sharing: groups of 8 sequences share the
    # 32 physical blocks of a 512-token prefix (refcount 8).
    "llama13b_prefix": DecodeConfig(
        name="llama13b_prefix", seed=3, num_seqs=64, num_heads=40, num_kv_heads=40, head_dim=128,
        block_size=16, num_blocks=16384, max_blocks_per_seq=256, kv_dtype="bf16", q_dtype="bf16",
        ctx_kind="uniform", ctx_lo=512, ctx_hi=4096, allocator="prefix",
        share_group=8, share_prefix_blocks=32,
    ),
    # 70B-shaped grouped-query decode: 64 query heads over 8 KV heads, block 32,
    # lognormal lengths, pool fragmented by an allocate/free churn simulation.
    "gqa70b": DecodeConfig(
        name="gqa70b", seed=4, num_seqs=128, num_heads=64, num_kv_heads=8, head_dim=128,
        block_size=32, num_blocks=40000, max_blocks_per_seq=256, kv_dtype="f16", q_dtype="f16",
        ctx_kind="lognormal", ctx_median=1024.0, ctx_sigma=1.0, ctx_lo=1, ctx_hi=8192,
        allocator="churn",
    ),
    # Long-context fp8-e4m3 KV with per-tensor scales, fp16 query, 512-token partitions.
    "fp8_long": DecodeConfig(
        name="fp8_long", seed=5, num_seqs=8, num_heads=32, num_kv_heads=32, head_dim=128,
        block_size=16, num_blocks=20480, max_blocks_per_seq=2048, kv_dtype="fp8", q_dtype="f16",
        ctx_kind="uniform", ctx_lo=16384, ctx_hi=32768, allocator="shuffled",
        partition_size=512,
    ),
    # The 70B-shaped grouped-query step with an fp8-e4m3 cache and one scale per
    # kv head (an fp8 KV cache on a 70B model, page "大模型推理KV Cache内存管理与
    # PagedAttention分页显存实战"; precision chosen per head, page "vLLM框架中的KV
    # cache优化与PagedAttention机制详解" section 8.2).  The kv heads' K/V values
    # range from std 1/4 to std 4, so one scale per tensor would leave the
    # quiet heads a few bits.
    "gqa70b_fp8": DecodeConfig(
        name="gqa70b_fp8", seed=6, num_seqs=128, num_heads=64, num_kv_heads=8, head_dim=128,
        block_size=32, num_blocks=40000, max_blocks_per_seq=256, kv_dtype="fp8", q_dtype="f16",
        ctx_kind="lognormal", ctx_median=1024.0, ctx_sigma=1.0, ctx_lo=1, ctx_hi=8192,
        allocator="churn", fp8_scales="head", head_std=(0.25, 4.0),
    ),
    # The same with one fp8 scale per (physical block, kv head): the grain of
    # the pool's own blocks, each scale fitted to what its block holds.
    "gqa70b_fp8_blocks": DecodeConfig(
        name="gqa70b_fp8_blocks", seed=6, num_seqs=128, num_heads=64, num_kv_heads=8, head_dim=128,
        block_size=32, num_blocks=40000, max_blocks_per_seq=256, kv_dtype="fp8", q_dtype="f16",
        ctx_kind="lognormal", ctx_median=1024.0, ctx_sigma=1.0, ctx_lo=1, ctx_hi=8192,
        allocator="churn", fp8_scales="block", head_std=(0.25, 4.0),
    ),
}

# the order the five workloads are listed in
CONFIG_ORDER = ("tiny", "llama7b", "llama13b_prefix", "gqa70b", "fp8_long")


def get_config(name: str) -> DecodeConfig:
    return CONFIGS[name]


def scaled(cfg: DecodeConfig, **overrides) -> DecodeConfig:
    """A copy of ``cfg`` with some fields replaced (smaller parity cases)."""
    return dataclasses.replace(cfg, **overrides)

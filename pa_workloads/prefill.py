"""Seeded workloads with several query tokens per sequence (paged prefill).

A prefill workload is a decode workload's shapes, pool and context-length
distribution plus a number of query tokens per sequence: the sequence's newest
q_len tokens (all of them if the context is shorter).  Their K/V rows are what
the step's cache write stores; every earlier position is already in the cache.
Nothing here computes attention: layouts, slots and seeded values only.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Tuple, Union

import numpy as np

from .configs import DecodeConfig
from .generate import (ELEM_BYTES, FP8_MAX, Layout, _fill_pool, _pool_masked_amax, block_scales, head_stds, make_layout,
                       torch_dtype)


@dataclass(frozen=True)
class PrefillConfig:
    name: str
    base: DecodeConfig  # heads, head_dim, block size, dtypes, pool, context lengths, placement
    q_len: Union[int, Tuple[int, ...]]  # query tokens per sequence (one value, or one per sequence)

    def q_lens(self, context_lens: np.ndarray) -> np.ndarray:
        S = self.base.num_seqs
        want = np.full(S, self.q_len, dtype=np.int64) if isinstance(self.q_len, int) else np.array(self.q_len)
        if want.shape != (S,):
            raise ValueError(f"{self.name}: one q_len per sequence expected")
        return np.minimum(want, np.asarray(context_lens, dtype=np.int64)).astype(np.int32)


PREFILL_CONFIGS: Dict[str, PrefillConfig] = {
    # Small grouped-query case for parity: three sequences, four query heads per
    # kv head, contexts of 5, 40 and 70 tokens of which 5, 17 and 33 are new.
    "prefill_small": PrefillConfig(
        name="prefill_small",
        base=DecodeConfig(
            name="prefill_small", seed=11, num_seqs=3, num_heads=8, num_kv_heads=2, head_dim=64,
            block_size=16, num_blocks=32, max_blocks_per_seq=6, kv_dtype="f16", q_dtype="f16",
            ctx_kind="fixed", ctx_fixed=(5, 40, 70), allocator="permutation",
        ),
        q_len=(5, 17, 33),
    ),
    # Chunked prefill on LLaMA-7B shapes: 512-token chunks of prompts whose
    # contexts (earlier chunks included) are uniform in [1024, 4096].
    "prefill_7b": PrefillConfig(
        name="prefill_7b",
        base=DecodeConfig(
            name="prefill_7b", seed=12, num_seqs=8, num_heads=32, num_kv_heads=32, head_dim=128,
            block_size=16, num_blocks=5000, max_blocks_per_seq=256, kv_dtype="f16", q_dtype="f16",
            ctx_kind="uniform", ctx_lo=1024, ctx_hi=4096, allocator="shuffled",
        ),
        q_len=512,
    ),
    # Speculative-decode verification on 70B grouped-query shapes: four draft
    # tokens per sequence over the gqa70b context-length distribution and pool.
    "verify_gqa70b": PrefillConfig(
        name="verify_gqa70b",
        base=DecodeConfig(
            name="verify_gqa70b", seed=13, num_seqs=128, num_heads=64, num_kv_heads=8, head_dim=128,
            block_size=32, num_blocks=40000, max_blocks_per_seq=256, kv_dtype="f16", q_dtype="f16",
            ctx_kind="lognormal", ctx_median=1024.0, ctx_sigma=1.0, ctx_lo=4, ctx_hi=8192, allocator="churn",
        ),
        q_len=4,
    ),
    # The same two steps over fp8 e4m3fn caches with per-tensor scales (the fp8
    # KV cache of page "大模型推理KV Cache内存管理与PagedAttention分页显存实战"),
    # f16 queries: half the cache bytes of the 16-bit steps.
    "prefill_7b_fp8": PrefillConfig(
        name="prefill_7b_fp8",
        base=DecodeConfig(
            name="prefill_7b_fp8", seed=14, num_seqs=8, num_heads=32, num_kv_heads=32, head_dim=128,
            block_size=16, num_blocks=5000, max_blocks_per_seq=256, kv_dtype="fp8", q_dtype="f16",
            ctx_kind="uniform", ctx_lo=1024, ctx_hi=4096, allocator="shuffled",
        ),
        q_len=512,
    ),
    "verify_gqa70b_fp8": PrefillConfig(
        name="verify_gqa70b_fp8",
        base=DecodeConfig(
            name="verify_gqa70b_fp8", seed=15, num_seqs=128, num_heads=64, num_kv_heads=8, head_dim=128,
            block_size=32, num_blocks=40000, max_blocks_per_seq=256, kv_dtype="fp8", q_dtype="f16",
            ctx_kind="lognormal", ctx_median=1024.0, ctx_sigma=1.0, ctx_lo=4, ctx_hi=8192, allocator="churn",
        ),
        q_len=4,
    ),
}


def get_prefill_config(name: str) -> PrefillConfig:
    return PREFILL_CONFIGS[name]


@dataclass
class PrefillLayout:
    layout: Layout  # context lengths, block tables (the decode layout of the base config)
    q_lens: np.ndarray  # int32 [S]
    query_start_loc: np.ndarray  # int32 [S + 1]
    slot_mapping: np.ndarray  # int64 [N]: slot of every new token, in query-row order

    def stored_mask(self) -> np.ndarray:
        """bool [num_blocks, block_size]: slots holding data before the step's cache write."""
        cfg = self.layout.cfg
        bs = cfg.block_size
        mask = np.zeros((cfg.num_blocks, bs), dtype=bool)
        for i in range(cfg.num_seqs):
            n_stored = int(self.layout.context_lens[i]) - int(self.q_lens[i])
            for j in range(-(-n_stored // bs)):
                mask[self.layout.block_tables[i, j], : min(bs, n_stored - j * bs)] = True
        return mask


def make_prefill_layout(pcfg: PrefillConfig) -> PrefillLayout:
    layout = make_layout(pcfg.base)
    if (layout.refcount > 1).any():
        raise ValueError("prefill workloads keep every block private (their new tokens are all written)")
    bs = pcfg.base.block_size
    q_lens = pcfg.q_lens(layout.context_lens)
    qsl = np.zeros(pcfg.base.num_seqs + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(q_lens)
    slots = np.empty(int(qsl[-1]), dtype=np.int64)
    for i in range(pcfg.base.num_seqs):
        ctx, nq = int(layout.context_lens[i]), int(q_lens[i])
        for j in range(nq):
            pos = ctx - nq + j
            slots[qsl[i] + j] = int(layout.block_tables[i, pos // bs]) * bs + pos % bs
    return PrefillLayout(layout, q_lens, qsl, slots)


def make_prefill_inputs(pcfg: PrefillConfig, pl: PrefillLayout, device="cpu", seed_offset: int = 0) -> dict:
    """q [N, H, D]; k_cache/v_cache with every position before the new tokens
    stored (the rest NaN, code 0x7F for fp8); k_new/v_new [N, Hkv, D]; int32
    context_lens, block_tables, query_start_loc; int64 slot_mapping [N];
    k_scale/v_scale: fp8 scales per tensor (floats; 1.0 for other dtypes), per
    kv head (float32 tensors [Hkv]) or per block (float32 tensors [num_blocks,
    Hkv]), as make_inputs draws them."""
    import torch

    cfg = pcfg.base
    N = int(pl.query_start_loc[-1])
    H, Hkv, D = cfg.num_heads, cfg.num_kv_heads, cfg.head_dim
    shape = (cfg.num_blocks, cfg.block_size, Hkv, D)
    base = cfg.seed * 1000 + seed_offset * 17
    chunk_blocks = max(1, (1 << 24) // (cfg.block_size * Hkv * D))
    mask_t = torch.from_numpy(pl.stored_mask()).to(device)
    gq = torch.Generator(device=device)
    gq.manual_seed(base + 1)
    q = torch.randn((N, H, D), generator=gq, device=device, dtype=torch.float32).to(torch_dtype(cfg.q_dtype))
    new_dtype = cfg.q_dtype if cfg.kv_dtype == "fp8" else cfg.kv_dtype
    std_t = torch.from_numpy(head_stds(cfg)).to(device).reshape(1, 1, Hkv, 1)
    gn = torch.Generator(device=device)
    gn.manual_seed(base + 4)
    k_new = (torch.randn((N, Hkv, D), generator=gn, device=device, dtype=torch.float32) * std_t[0]) \
        .to(torch_dtype(new_dtype))
    v_new = (torch.randn((N, Hkv, D), generator=gn, device=device, dtype=torch.float32) * std_t[0]) \
        .to(torch_dtype(new_dtype))
    k_scale = v_scale = 1.0
    k_q = v_q = None
    if cfg.kv_dtype == "fp8":
        ka = torch.maximum(_pool_masked_amax(shape, base + 2, mask_t, device, chunk_blocks, std_t),
                           k_new.float().abs().amax(dim=(0, 2))).cpu().numpy().astype(np.float64)
        va = torch.maximum(_pool_masked_amax(shape, base + 3, mask_t, device, chunk_blocks, std_t),
                           v_new.float().abs().amax(dim=(0, 2))).cpu().numpy().astype(np.float64)
        if cfg.fp8_scales == "block":  # one scale per (block, kv head), float32 tensors [num_blocks, Hkv]
            k_scale, v_scale = block_scales(cfg, base, k_new, v_new, pl.slot_mapping, mask_t, device, std_t)
            k_q = k_scale.reshape(cfg.num_blocks, 1, Hkv, 1)
            v_q = v_scale.reshape(cfg.num_blocks, 1, Hkv, 1)
        elif cfg.fp8_scales == "head":  # one scale per kv head, float32 tensors [Hkv]
            k_scale = torch.from_numpy((ka / FP8_MAX * (1.0 + 2.0**-16)).astype(np.float32)).to(device)
            v_scale = torch.from_numpy((va / FP8_MAX * (1.0 + 2.0**-16)).astype(np.float32)).to(device)
            k_q, v_q = k_scale.reshape(1, 1, Hkv, 1), v_scale.reshape(1, 1, Hkv, 1)
        else:
            k_scale = float(np.float32(ka.max() / FP8_MAX * (1.0 + 2.0**-16)))
            v_scale = float(np.float32(va.max() / FP8_MAX * (1.0 + 2.0**-16)))
            k_q, v_q = k_scale, v_scale
    k_cache = _fill_pool(shape, cfg.kv_dtype, base + 2, mask_t, device, chunk_blocks, std_t, k_q)
    v_cache = _fill_pool(shape, cfg.kv_dtype, base + 3, mask_t, device, chunk_blocks, std_t, v_q)
    L = pl.layout
    return {
        "q": q,
        "k_cache": k_cache,
        "v_cache": v_cache,
        "k_new": k_new,
        "v_new": v_new,
        "k_scale": k_scale,
        "v_scale": v_scale,
        "context_lens": torch.from_numpy(L.context_lens.copy()).to(device),
        "block_tables": torch.from_numpy(L.block_tables.copy()).to(device),
        "query_start_loc": torch.from_numpy(pl.query_start_loc.copy()).to(device),
        "slot_mapping": torch.from_numpy(pl.slot_mapping.copy()).to(device),
    }


def prefill_flops(pcfg: PrefillConfig, pl: PrefillLayout) -> int:
    """Algorithmic flops of a prefill launch: 4 D per (query row, head, visible key)."""
    cfg = pcfg.base
    total = 0
    for i in range(cfg.num_seqs):
        ctx, nq = int(pl.layout.context_lens[i]), int(pl.q_lens[i])
        # query j sees ctx - nq + j + 1 keys
        total += nq * (ctx - nq) + nq * (nq + 1) // 2
    return 4 * cfg.head_dim * cfg.num_heads * total


def prefill_kv_bytes(pcfg: PrefillConfig, pl: PrefillLayout) -> int:
    """K and V bytes of every context token, read once per (sequence, kv head)."""
    cfg = pcfg.base
    return int(2 * int(pl.layout.context_lens.astype(np.int64).sum()) * cfg.num_kv_heads * cfg.head_dim
               * ELEM_BYTES[cfg.kv_dtype])


def prefill_algorithmic_bytes(pcfg: PrefillConfig, pl: PrefillLayout) -> int:
    """Bytes a prefill launch must move at least: every context K/V row once per
    (sequence, kv head), the queries, the outputs (query dtype), the block-table
    entries it reads, the context lengths and query offsets."""
    cfg = pcfg.base
    N = int(pl.query_start_loc[-1])
    ctx = pl.layout.context_lens.astype(np.int64)
    eq = ELEM_BYTES[cfg.q_dtype]
    return int(prefill_kv_bytes(pcfg, pl) + 2 * N * cfg.num_heads * cfg.head_dim * eq
               + 4 * int(np.sum(-(-ctx // cfg.block_size))) + 4 * (2 * cfg.num_seqs + 1))

"""Seeded workloads for whole-block copies: copy-on-write inside one device
pool, and swapping blocks out to / in from a pinned host pool.

Only layouts and values are drawn here (which blocks move where, the pool's
bytes); nothing is copied.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Dict

import numpy as np

from .configs import DecodeConfig, get_config, scaled
from .generate import ELEM_BYTES, torch_dtype


@dataclass(frozen=True)
class BlockCopyConfig:
    name: str
    base: DecodeConfig  # block shape, dtype and device pool size
    num_pairs: int
    kind: str  # "cow" (device -> same device pool) | "swap_out" (device -> host) | "swap_in" (host -> device)
    seed: int

    @property
    def block_bytes(self) -> int:
        b = self.base
        return b.block_size * b.num_kv_heads * b.head_dim * ELEM_BYTES[b.kv_dtype]

    def bytes_moved(self) -> int:
        """K and V bytes read plus bytes written by one launch (every pair valid)."""
        return 2 * 2 * self.num_pairs * self.block_bytes


BLOCK_CONFIGS: Dict[str, BlockCopyConfig] = {
    # a batch of 32 beams forking at once, each taking private copies of 32
    # shared blocks (512 tokens) of a 7B-shaped fp16 pool before writing
    "cow_llama7b": BlockCopyConfig("cow_llama7b", get_config("llama7b"), num_pairs=1024, kind="cow", seed=21),
    # preemption: 32 sequences of 2048 tokens of the 70B-shaped pool leave for
    # host memory (64 blocks of 32 tokens each), and come back elsewhere
    "swap_out_gqa70b": BlockCopyConfig("swap_out_gqa70b", get_config("gqa70b"), num_pairs=2048, kind="swap_out",
                                       seed=22),
    "swap_in_gqa70b": BlockCopyConfig("swap_in_gqa70b", get_config("gqa70b"), num_pairs=2048, kind="swap_in",
                                      seed=23),
    # small cases for parity
    "cow_small_bf16": BlockCopyConfig("cow_small_bf16", scaled(get_config("llama13b_prefix"), num_blocks=300,
                                                               num_kv_heads=4, num_heads=4),
                                      num_pairs=37, kind="cow", seed=24),
    "swap_small_fp8": BlockCopyConfig("swap_small_fp8", scaled(get_config("fp8_long"), num_blocks=200, num_kv_heads=2,
                                                               num_heads=2, head_dim=64),
                                      num_pairs=45, kind="swap_out", seed=25),
}


def block_mapping(cfg: BlockCopyConfig) -> np.ndarray:
    """int64 [M, 2] (source, destination), drawn from the config's seed.
    cow: distinct sources and distinct destinations, disjoint, in one pool.
    swap_out: distinct device sources, destinations 0 .. M-1 of the host pool.
    swap_in: sources 0 .. M-1 of the host pool, distinct device destinations."""
    rng = np.random.Generator(np.random.PCG64(cfg.seed))
    nb, M = cfg.base.num_blocks, cfg.num_pairs
    if cfg.kind == "cow":
        ids = rng.permutation(nb)[: 2 * M]
        return np.stack([ids[:M], ids[M:]], axis=1).astype(np.int64)
    dev = rng.permutation(nb)[:M]
    host = np.arange(M)
    if cfg.kind == "swap_out":
        return np.stack([dev, host], axis=1).astype(np.int64)
    if cfg.kind == "swap_in":
        return np.stack([host, dev], axis=1).astype(np.int64)
    raise ValueError(cfg.kind)


def pool_shapes(cfg: BlockCopyConfig):
    """(source pool shape, destination pool shape, source on host?, destination on host?)"""
    b = cfg.base
    dev = (b.num_blocks, b.block_size, b.num_kv_heads, b.head_dim)
    host = (cfg.num_pairs, b.block_size, b.num_kv_heads, b.head_dim)
    if cfg.kind == "cow":
        return dev, dev, False, False
    if cfg.kind == "swap_out":
        return dev, host, False, True
    return host, dev, True, False


def random_pool(shape, kv_dtype: str, seed: int, device="cpu", pin: bool = False):
    """A pool filled with seeded N(0,1) values in its storage dtype (fp8 codes
    are drawn as raw finite bytes: every code except the two NaNs), drawn on
    ``device`` (a pinned pool is drawn on the CPU)."""
    import torch

    dev = "cpu" if pin else device
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    if kv_dtype == "fp8":
        codes = torch.randint(0, 254, shape, generator=g, dtype=torch.int32, device=dev)
        codes = codes + (codes >= 0x7F).to(torch.int32)  # skip 0x7F: NaN codes are 0x7F and 0xFF
        t = codes.to(torch.uint8).view(torch.float8_e4m3fn)
    else:
        t = torch.randn(shape, generator=g, dtype=torch.float32, device=dev).to(torch_dtype(kv_dtype))
    return t.pin_memory() if pin else t

"""Seeded multi-layer decode workloads: L layers of one decode workload that
share its layout (context lengths, block tables, the new token's slots) and
each draw their own queries, caches and new K/V rows.  Nothing is computed
here."""

from __future__ import annotations

from dataclasses import dataclass
from typing import Dict

from .configs import DecodeConfig, get_config
from .generate import Layout, make_inputs


@dataclass(frozen=True)
class LayerConfig:
    name: str
    base: DecodeConfig
    num_layers: int


LAYER_CONFIGS: Dict[str, LayerConfig] = {
    # eight layers of the 7B-shaped fp16 decode step (4.2 GB of K/V per step)
    "llama7b_x8": LayerConfig("llama7b_x8", get_config("llama7b"), 8),
    # eight layers of the 70B-shaped grouped-query step (7.2 GB)
    "gqa70b_x8": LayerConfig("gqa70b_x8", get_config("gqa70b"), 8),
}


def make_layer_inputs(lcfg: LayerConfig, layout: Layout, device="cpu", seed_offset: int = 0) -> dict:
    """Per-layer tensors stacked on a leading layer dimension: q [L, S, H, D],
    k_cache / v_cache [L, NB, bs, Hkv, D], k_new / v_new [L, S, Hkv, D]; the
    shared int32 context_lens [S], block_tables [S, W] and int64 slot_mapping
    [S]; fp8 scales (the first layer's; the workloads here are 16-bit)."""
    import torch

    L = lcfg.num_layers
    out = None
    for l in range(L):
        inp = make_inputs(lcfg.base, layout, device, seed_offset=1000 * seed_offset + l)
        if out is None:
            out = {k: (torch.empty((L,) + tuple(v.shape), dtype=v.dtype, device=v.device)
                       if k in ("q", "k_cache", "v_cache", "k_new", "v_new") else v) for k, v in inp.items()}
        for k in ("q", "k_cache", "v_cache", "k_new", "v_new"):
            out[k][l].copy_(inp[k])
        del inp
    return out


def flat_slots(slot_mapping, num_layers: int, slots_per_layer: int):
    """The slots of every layer's new rows in the pools flattened to
    [L * NB, bs, ...]: layer l's slot s becomes l * NB * bs + s (negative stays
    negative, i.e. skipped)."""
    import torch

    sm = slot_mapping.to(torch.int64)
    offs = torch.arange(num_layers, device=sm.device, dtype=torch.int64).unsqueeze(1) * slots_per_layer
    return torch.where(sm.unsqueeze(0) >= 0, sm.unsqueeze(0) + offs, sm.unsqueeze(0)).reshape(-1).contiguous()

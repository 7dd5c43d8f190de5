"""Seeded synthetic inputs for paged-KV decode.

This package only *draws* inputs: context lengths, block tables produced by a
few block allocators, slot mappings for the newly appended token of every
sequence, and random query / key / value data with every unread slot poisoned.
It holds none of the attention arithmetic; both the HIP path and the CPU oracle
consume what it produces, and neither imports the other.

The shapes follow the workloads the pages name (LLaMA-7B / 13B / 70B-style
heads, block sizes 16 and 32, ragged context lengths; see the pages
"vLLM推理引擎架构：PagedAttention机制与高吞吐推理" section 2.2 for the cache layout
and "大模型推理KV Cache内存管理与PagedAttention分页显存实战" for block size 16/32
and the model shapes).
"""

from .configs import CONFIGS, DecodeConfig, get_config, scaled
from .generate import Layout, make_layout, make_inputs, kv_bytes, algorithmic_bytes

__all__ = [
    "CONFIGS",
    "DecodeConfig",
    "get_config",
    "scaled",
    "Layout",
    "make_layout",
    "make_inputs",
    "kv_bytes",
    "algorithmic_bytes",
]

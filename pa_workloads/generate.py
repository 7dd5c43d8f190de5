"""Seeded layouts (context lengths, block tables, slot mappings) and input tensors.

Layouts are drawn with numpy's PCG64 generator.  Value tensors are drawn with a
seeded torch generator on the device that will hold them (torch's CPU generator
on the host, its Philox generator on a GPU), so full-size caches take
milliseconds to fill.  Both sides of every comparison read the same stored
bytes, so the two generators never need to agree with each other.

Every cache slot that no sequence reads (slots of unreferenced blocks, the tail
of each sequence's last block, the whole trap block that pads the tables) is
filled with NaN (code 0x7F for fp8), so a kernel that reads one shows it.
"""

from __future__ import annotations

import collections
import math
from dataclasses import dataclass, field
from typing import Dict, List

import numpy as np

from .configs import DecodeConfig

FP8_MAX = 448.0
FP8_NAN_CODE = 0x7F

ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1}


@dataclass
class Layout:
    cfg: DecodeConfig
    context_lens: np.ndarray  # int32 [S]
    block_tables: np.ndarray  # int32 [S, W]; entries past a sequence's blocks hold trap_block
    num_valid_blocks: np.ndarray  # int32 [S] = ceil(ctx / block_size)
    slot_mapping: np.ndarray  # int64 [S]; slot of each sequence's last token, -1 if already stored
    refcount: np.ndarray  # int32 [num_blocks]
    trap_block: int
    stats: Dict[str, float] = field(default_factory=dict)

    @property
    def new_positions(self) -> np.ndarray:
        return self.context_lens.astype(np.int64) - 1

    def stored_mask(self) -> np.ndarray:
        """bool [num_blocks, block_size]: slots holding data before the cache write.

        A sequence's positions 0 .. ctx-2 are stored; its last position (ctx-1) is
        stored too when it lies in a shared block (slot_mapping == -1), and is
        otherwise left for the cache write.
        """
        cfg = self.cfg
        bs = cfg.block_size
        mask = np.zeros((cfg.num_blocks, bs), dtype=bool)
        for i in range(cfg.num_seqs):
            ctx = int(self.context_lens[i])
            n_stored = ctx - 1 if self.slot_mapping[i] >= 0 else ctx
            for j in range(int(self.num_valid_blocks[i])):
                lo = j * bs
                cnt = min(bs, n_stored - lo)
                if cnt > 0:
                    mask[self.block_tables[i, j], :cnt] = True
        return mask


def _draw_context_lens(cfg: DecodeConfig, rng: np.random.Generator) -> np.ndarray:
    if cfg.ctx_kind == "fixed":
        ctx = np.array(cfg.ctx_fixed, dtype=np.int64)
        assert ctx.shape[0] == cfg.num_seqs
    elif cfg.ctx_kind == "uniform":
        ctx = rng.integers(cfg.ctx_lo, cfg.ctx_hi + 1, size=cfg.num_seqs)
    elif cfg.ctx_kind == "lognormal":
        raw = np.exp(rng.normal(math.log(cfg.ctx_median), cfg.ctx_sigma, size=cfg.num_seqs))
        ctx = np.clip(np.rint(raw), cfg.ctx_lo, cfg.ctx_hi).astype(np.int64)
    else:
        raise ValueError(cfg.ctx_kind)
    return ctx.astype(np.int32)


def _alloc_front(free: collections.deque, n: int) -> List[int]:
    # allocation takes from the front of the free list, freeing appends to its end
    # (page "vLLM推理引擎架构：PagedAttention机制与高吞吐推理", section 2.2)
    if len(free) < n:
        raise MemoryError(f"need {n} blocks, only {len(free)} available")
    return [free.popleft() for _ in range(n)]


def _churn(cfg: DecodeConfig, need: np.ndarray, rng: np.random.Generator):
    """Allocate the measured sequences while background sequences come and go.

    Background sequences are admitted (same length law as the measured ones),
    grown by one block, or freed, keeping pool occupancy inside ``churn_band``.
    The measured sequences grow one block per round, round-robin, interleaved
    with the churn, the way decode grows sequences a block at a time.
    """
    nb = cfg.num_blocks
    lo, hi = cfg.churn_band
    free = collections.deque(range(nb))
    background: Dict[int, List[int]] = {}
    next_id = 0
    measured: List[List[int]] = [[] for _ in range(cfg.num_seqs)]
    remaining = int(need.sum())

    def bg_len_blocks() -> int:
        raw = math.exp(rng.normal(math.log(max(cfg.ctx_median, 1.0)), max(cfg.ctx_sigma, 1e-9)))
        ctx = int(np.clip(round(raw), cfg.ctx_lo, cfg.ctx_hi))
        return -(-ctx // cfg.block_size)

    def free_random_bg() -> bool:
        if not background:
            return False
        keys = sorted(background)
        k = keys[int(rng.integers(len(keys)))]
        free.extend(background.pop(k))
        return True

    # warm the pool up to the low edge of the band
    while (nb - len(free)) < lo * nb:
        n = bg_len_blocks()
        if len(free) - n < remaining:
            break
        background[next_id] = _alloc_front(free, n)
        next_id += 1

    rounds = int(need.max()) if need.size else 0
    for _ in range(rounds):
        for i in range(cfg.num_seqs):
            if len(measured[i]) < need[i]:
                while len(free) < 1 and free_random_bg():
                    pass
                measured[i].extend(_alloc_front(free, 1))
                remaining -= 1
        for _ in range(4):
            occ = (nb - len(free)) / nb
            if occ < lo:
                op = 0
            elif occ > hi:
                op = 2
            else:
                op = int(rng.choice(3, p=[0.3, 0.4, 0.3]))
            if op == 0:
                n = bg_len_blocks()
                if len(free) - n >= remaining:
                    background[next_id] = _alloc_front(free, n)
                    next_id += 1
                else:
                    free_random_bg()
            elif op == 1 and background:
                if len(free) - 1 >= remaining:
                    keys = sorted(background)
                    k = keys[int(rng.integers(len(keys)))]
                    background[k].extend(_alloc_front(free, 1))
                else:
                    free_random_bg()
            else:
                free_random_bg()
    occupancy = (nb - len(free)) / nb
    return measured, list(free), occupancy


def make_layout(cfg: DecodeConfig) -> Layout:
    rng = np.random.Generator(np.random.PCG64(cfg.seed))
    S, W, bs, NB = cfg.num_seqs, cfg.max_blocks_per_seq, cfg.block_size, cfg.num_blocks
    ctx = _draw_context_lens(cfg, rng)
    if (ctx < 1).any():
        raise ValueError("every sequence holds at least its new token")
    need = -(-ctx.astype(np.int64) // bs)
    if need.max() > W:
        raise ValueError(f"{cfg.name}: a sequence needs {need.max()} blocks > table width {W}")
    refcount = np.zeros(NB, dtype=np.int32)
    tables: List[List[int]] = []
    free_after: List[int]
    occupancy = float("nan")

    if cfg.allocator in ("permutation", "shuffled"):
        # a seeded shuffled free list, taken from the front sequence by sequence
        free = collections.deque(int(b) for b in rng.permutation(NB))
        for i in range(S):
            tables.append(_alloc_front(free, int(need[i])))
        free_after = list(free)
    elif cfg.allocator == "prefix":
        free = collections.deque(int(b) for b in rng.permutation(NB))
        P = cfg.share_prefix_blocks
        if (need < P).any():
            raise ValueError("every sequence must cover the shared prefix")
        for g0 in range(0, S, cfg.share_group):
            prefix = _alloc_front(free, P)
            for i in range(g0, min(S, g0 + cfg.share_group)):
                tables.append(prefix + _alloc_front(free, int(need[i]) - P))
        free_after = list(free)
    elif cfg.allocator == "churn":
        tables, free_after, occupancy = _churn(cfg, need, rng)
    else:
        raise ValueError(cfg.allocator)

    for t in tables:
        for b in t:
            refcount[b] += 1
    unreferenced = [b for b in free_after if refcount[b] == 0]
    if not unreferenced:
        unreferenced = [int(b) for b in np.nonzero(refcount == 0)[0]]
    if not unreferenced:
        raise ValueError(f"{cfg.name}: pool too small to keep a trap block")
    trap = int(unreferenced[0])

    bt = np.full((S, W), trap, dtype=np.int32)
    for i, t in enumerate(tables):
        bt[i, : len(t)] = t
    slot = np.empty(S, dtype=np.int64)
    for i in range(S):
        pos = int(ctx[i]) - 1
        blk = int(bt[i, pos // bs])
        # a token whose block is shared was stored by the prefix's writer: skip it
        slot[i] = -1 if refcount[blk] > 1 else blk * bs + pos % bs

    pairs = 0
    breaks = 0
    for t in tables:
        for a, b in zip(t[:-1], t[1:]):
            pairs += 1
            breaks += int(b != a + 1)
    stats = {
        "blocks_referenced": int((refcount > 0).sum()),
        "block_refs": int(refcount.sum()),
        "non_adjacent_fraction": breaks / pairs if pairs else 0.0,
        "pool_occupancy_after_churn": occupancy,
        "mean_ctx": float(ctx.mean()),
    }
    return Layout(cfg, ctx, bt, need.astype(np.int32), slot, refcount, trap, stats)


# ----------------------------------------------------------------------------------------
# value tensors

def torch_dtype(name: str):
    import torch

    return {
        "f32": torch.float32,
        "f16": torch.float16,
        "bf16": torch.bfloat16,
        "fp8": torch.float8_e4m3fn,
    }[name]


def head_stds(cfg: DecodeConfig) -> np.ndarray:
    """float32 [num_kv_heads]: the standard deviation of each kv head's K and V
    values (geometric from cfg.head_std[0] to cfg.head_std[1])."""
    lo, hi = cfg.head_std
    n = cfg.num_kv_heads
    return np.geomspace(lo, hi, n).astype(np.float32) if n > 1 else np.array([lo], dtype=np.float32)


def _pool_masked_amax(shape, gen_seed, mask_t, device, chunk_blocks, std_t):
    """float32 [num_kv_heads]: the largest stored magnitude of each kv head."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(gen_seed)
    amax = torch.zeros((shape[2],), dtype=torch.float32, device=device)
    for b0 in range(0, shape[0], chunk_blocks):
        b1 = min(shape[0], b0 + chunk_blocks)
        x = torch.randn((b1 - b0,) + tuple(shape[1:]), generator=g, device=device, dtype=torch.float32) * std_t
        m = mask_t[b0:b1, :, None, None]
        amax = torch.maximum(amax, torch.where(m, x.abs(), torch.zeros_like(x)).amax(dim=(0, 1, 3)))
    return amax


def _pool_masked_block_amax(shape, gen_seed, mask_t, device, chunk_blocks, std_t):
    """float32 [num_blocks, num_kv_heads]: the largest stored magnitude of each
    (block, kv head) -- the same draws as _fill_pool."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(gen_seed)
    amax = torch.zeros((shape[0], shape[2]), dtype=torch.float32, device=device)
    for b0 in range(0, shape[0], chunk_blocks):
        b1 = min(shape[0], b0 + chunk_blocks)
        x = torch.randn((b1 - b0,) + tuple(shape[1:]), generator=g, device=device, dtype=torch.float32) * std_t
        m = mask_t[b0:b1, :, None, None]
        amax[b0:b1] = torch.where(m, x.abs(), torch.zeros_like(x)).amax(dim=(1, 3))
    return amax


def block_scales(cfg, base, k_new, v_new, slot_mapping, mask_t, device, std_t):
    """float32 [num_blocks, num_kv_heads] key and value scales, one per (block,
    kv head): the largest magnitude the block holds for that head -- its
    stored values and the new rows whose slots lie in it -- maps just under
    448; a block with nothing stored gets a thousandth of its head's std."""
    import torch

    Hkv = cfg.num_kv_heads
    shape = (cfg.num_blocks, cfg.block_size, Hkv, cfg.head_dim)
    chunk_blocks = max(1, (1 << 24) // (cfg.block_size * Hkv * cfg.head_dim))
    out = []
    for seed, new in ((base + 2, k_new), (base + 3, v_new)):
        am = _pool_masked_block_amax(shape, seed, mask_t, device, chunk_blocks, std_t)
        slot = torch.from_numpy(np.asarray(slot_mapping).copy()).to(device)
        live = slot >= 0
        if bool(live.any()):  # the new rows land in their slot's block
            dst = (slot[live] // cfg.block_size).long()
            am.scatter_reduce_(0, dst[:, None].expand(-1, Hkv), new.float().abs().amax(dim=2)[live], "amax")
        am = torch.maximum(am, 1e-3 * std_t.reshape(1, Hkv))
        out.append((am.double() / FP8_MAX * (1.0 + 2.0**-16)).to(torch.float32))
    return out[0], out[1]


def _fill_pool(shape, dtype_name, gen_seed, mask_t, device, chunk_blocks, std_t, quant_scale=None):
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(gen_seed)
    out = torch.empty(shape, dtype=torch_dtype(dtype_name), device=device)
    for b0 in range(0, shape[0], chunk_blocks):
        b1 = min(shape[0], b0 + chunk_blocks)
        x = torch.randn((b1 - b0,) + tuple(shape[1:]), generator=g, device=device, dtype=torch.float32) * std_t
        m = mask_t[b0:b1, :, None, None].expand_as(x)
        if dtype_name == "fp8":
            qs = quant_scale
            if torch.is_tensor(qs) and qs.dim() == 4 and qs.shape[0] == shape[0]:  # per block: this chunk's
                qs = qs[b0:b1]
            codes = (x / qs).to(torch.float8_e4m3fn).view(torch.uint8)
            codes = torch.where(m, codes, torch.full_like(codes, FP8_NAN_CODE))
            out[b0:b1] = codes.view(torch.float8_e4m3fn)
        else:
            y = x.to(torch_dtype(dtype_name))
            out[b0:b1] = torch.where(m, y, torch.full_like(y, float("nan")))
    return out


def make_inputs(cfg: DecodeConfig, layout: Layout, device="cpu", seed_offset: int = 0) -> dict:
    """Draw q, both caches (poisoned where unread) and the new tokens' K/V.

    Returns torch tensors on ``device``: q [S,H,D]; k_cache/v_cache
    [num_blocks, block_size, Hkv, D]; k_new/v_new [S, Hkv, D]; int32
    context_lens and block_tables; int64 slot_mapping; plus k_scale/v_scale:
    per-tensor fp8 scales (floats; 1.0 for other dtypes), or for workloads with
    per-head fp8 scales float32 tensors [Hkv] on ``device`` (per-block:
    [num_blocks, Hkv]).  fp8 scales are chosen so the largest stored magnitude
    of the tensor (or of the kv head, or of the block's kv head), new tokens
    included, maps just under 448; a block with nothing stored gets the scale
    of a thousandth of its head's std.  Kv head h's values are N(0, 1) times
    head_stds(cfg)[h].
    """
    import torch

    S, H, Hkv, D = cfg.num_seqs, cfg.num_heads, cfg.num_kv_heads, cfg.head_dim
    shape = (cfg.num_blocks, cfg.block_size, Hkv, D)
    base = cfg.seed * 1000 + seed_offset * 17
    chunk_blocks = max(1, (1 << 24) // (cfg.block_size * Hkv * D))
    mask_t = torch.from_numpy(layout.stored_mask()).to(device)

    gq = torch.Generator(device=device)
    gq.manual_seed(base + 1)
    q = torch.randn((S, H, D), generator=gq, device=device, dtype=torch.float32).to(torch_dtype(cfg.q_dtype))
    new_dtype = cfg.q_dtype if cfg.kv_dtype == "fp8" else cfg.kv_dtype
    std_np = head_stds(cfg)
    std_t = torch.from_numpy(std_np).to(device).reshape(1, 1, Hkv, 1)
    gn = torch.Generator(device=device)
    gn.manual_seed(base + 4)
    k_new = (torch.randn((S, Hkv, D), generator=gn, device=device, dtype=torch.float32) * std_t[0]) \
        .to(torch_dtype(new_dtype))
    v_new = (torch.randn((S, Hkv, D), generator=gn, device=device, dtype=torch.float32) * std_t[0]) \
        .to(torch_dtype(new_dtype))

    k_scale = v_scale = 1.0
    k_q = v_q = None  # what the pool's values are divided by before encoding
    if cfg.kv_dtype == "fp8":
        ka = torch.maximum(_pool_masked_amax(shape, base + 2, mask_t, device, chunk_blocks, std_t),
                           k_new.float().abs().amax(dim=(0, 2))).cpu().numpy().astype(np.float64)
        va = torch.maximum(_pool_masked_amax(shape, base + 3, mask_t, device, chunk_blocks, std_t),
                           v_new.float().abs().amax(dim=(0, 2))).cpu().numpy().astype(np.float64)
        # float32 scales, nudged up so that |x| / scale stays below 448 after rounding
        if cfg.fp8_scales == "head":
            kh = (ka / FP8_MAX * (1.0 + 2.0**-16)).astype(np.float32)
            vh = (va / FP8_MAX * (1.0 + 2.0**-16)).astype(np.float32)
            k_scale = torch.from_numpy(kh).to(device)
            v_scale = torch.from_numpy(vh).to(device)
            k_q, v_q = k_scale.reshape(1, 1, Hkv, 1), v_scale.reshape(1, 1, Hkv, 1)
        elif cfg.fp8_scales == "block":
            k_scale, v_scale = block_scales(cfg, base, k_new, v_new, layout.slot_mapping, mask_t, device, std_t)
            k_q, v_q = k_scale.reshape(cfg.num_blocks, 1, Hkv, 1), v_scale.reshape(cfg.num_blocks, 1, Hkv, 1)
        elif cfg.fp8_scales == "tensor":
            k_scale = float(np.float32(ka.max() / FP8_MAX * (1.0 + 2.0**-16)))
            v_scale = float(np.float32(va.max() / FP8_MAX * (1.0 + 2.0**-16)))
            k_q, v_q = k_scale, v_scale
        else:
            raise ValueError(cfg.fp8_scales)
    k_cache = _fill_pool(shape, cfg.kv_dtype, base + 2, mask_t, device, chunk_blocks, std_t, k_q)
    v_cache = _fill_pool(shape, cfg.kv_dtype, base + 3, mask_t, device, chunk_blocks, std_t, v_q)

    return {
        "q": q,
        "k_cache": k_cache,
        "v_cache": v_cache,
        "k_new": k_new,
        "v_new": v_new,
        "k_scale": k_scale,
        "v_scale": v_scale,
        "context_lens": torch.from_numpy(layout.context_lens.copy()).to(device),
        "block_tables": torch.from_numpy(layout.block_tables.copy()).to(device),
        "slot_mapping": torch.from_numpy(layout.slot_mapping.copy()).to(device),
    }


# ----------------------------------------------------------------------------------------
# byte accounting (what a decode step must move at the least)

def kv_bytes(cfg: DecodeConfig, context_lens: np.ndarray) -> int:
    """K and V bytes of every valid token, read once each (logical, shared blocks counted per reader)."""
    return int(2 * int(np.asarray(context_lens, dtype=np.int64).sum()) * cfg.num_kv_heads * cfg.head_dim
               * ELEM_BYTES[cfg.kv_dtype])


def algorithmic_bytes(cfg: DecodeConfig, context_lens: np.ndarray, out_dtype: str = None) -> int:
    """Bytes a decode launch must move: K/V of valid tokens, q, out, table entries, lengths."""
    ctx = np.asarray(context_lens, dtype=np.int64)
    out_dtype = out_dtype or cfg.q_dtype
    S, H, D = cfg.num_seqs, cfg.num_heads, cfg.head_dim
    table = 4 * int((-(-ctx // cfg.block_size)).sum())
    head_scales = 2 * 4 * cfg.num_kv_heads if (cfg.kv_dtype == "fp8" and cfg.fp8_scales == "head") else 0
    # per-block scales: a key and a value scale per table entry read and kv head
    block_scales = 2 * cfg.num_kv_heads * table if (cfg.kv_dtype == "fp8" and cfg.fp8_scales == "block") else 0
    return (kv_bytes(cfg, ctx) + S * H * D * (ELEM_BYTES[cfg.q_dtype] + ELEM_BYTES[out_dtype])
            + table + 4 * S + head_scales + block_scales)

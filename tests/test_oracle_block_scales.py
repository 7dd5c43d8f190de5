"""Pins of the oracle's per-block fp8 scales: one scale per (physical block, kv
head), the finer grain of the precision per attention head of section 8.2 of
page "vLLM框架中的KV cache优化与PagedAttention机制详解", applied to the fp8 KV cache
of page "大模型推理KV Cache内存管理与PagedAttention分页显存实战": a token's stored
value is its code times the scale of the block that holds it, for its head.

Each check rests on something other than the oracle itself: torch's own fp8
casts with numpy/scipy attention (tokens dequantised with their own block's
scale, looked up through the block table in numpy), the already-pinned
per-head oracle, or an exact power-of-two identity.  Blocks and heads all get
distinct scales, so reading a neighbouring block's scale, the logical block
index instead of the physical one, or the wrong head's fails one of them.
"""

import numpy as np
import pytest
import torch

import oracle
from tests.test_oracle import paginate
from tests.textbook import attention, to_f64

SM_SCALE = 0.125


def _setup(G, seed=21, lens=(1, 15, 16, 17, 50, 97), Hkv=3, D=32, bs=16, shuffle=True):
    """fp8 rows with values drawn per (block, head) magnitude, blocks handed out
    in a shuffled order; returns the pool, tables and [NB, Hkv] block scales."""
    g = torch.Generator().manual_seed(seed)
    nb = sum(-(-L // bs) for L in lens) + 2
    order = torch.randperm(nb, generator=g).tolist() if shuffle else list(range(nb))
    # one magnitude per (physical block, head); scales near magnitude * 4.5 / 448
    mag = torch.exp(torch.randn((nb, Hkv), generator=g))
    k_bs = (mag * 4.5 / 448.0 * (1.0 + 0.1 * torch.rand((nb, Hkv), generator=g))).to(torch.float32)
    v_bs = (mag * 4.5 / 448.0 * (1.0 + 0.1 * torch.rand((nb, Hkv), generator=g))).to(torch.float32)
    rows, nxt = [], 0
    for L in lens:
        nblk = -(-L // bs)
        phys = order[nxt:nxt + nblk]
        nxt += nblk
        tok_blk = torch.tensor([phys[t // bs] for t in range(L)], dtype=torch.long)
        K = torch.randn((L, Hkv, D), generator=g) * mag[tok_blk][:, :, None]
        V = torch.randn((L, Hkv, D), generator=g) * mag[tok_blk][:, :, None]
        rows.append(((K / k_bs[tok_blk][:, :, None]).clamp(-448, 448).to(torch.float8_e4m3fn),
                     (V / v_bs[tok_blk][:, :, None]).clamp(-448, 448).to(torch.float8_e4m3fn)))
    q = torch.randn((len(lens), Hkv * G, D), generator=g).to(torch.float16)
    kc, vc, bt, ctx = paginate(rows, bs, nb, "fp8", order=order)
    return q, rows, kc, vc, bt, ctx, k_bs, v_bs, Hkv, bs


def _dequant_rows(rows, bt, bs, k_bs, v_bs):
    """(K, V) float64 per sequence: each token's codes (torch's decode) times its
    physical block's scale for that head, found through the table in numpy."""
    out = []
    for i, (K, V) in enumerate(rows):
        L = K.shape[0]
        phys = bt[i, np.arange(L) // bs].numpy()
        ks = k_bs.double().numpy()[phys][:, :, None]
        vs = v_bs.double().numpy()[phys][:, :, None]
        out.append((to_f64(K) * ks, to_f64(V) * vs))
    return out


@pytest.mark.parametrize("G", [1, 4])
def test_paged_decode_equals_textbook_with_block_scales(G):
    q, rows, kc, vc, bt, ctx, k_bs, v_bs, Hkv, bs = _setup(G)
    got = oracle.paged_decode(q, kc, vc, bt, ctx, SM_SCALE, Hkv, k_bs, v_bs)
    want = np.stack([attention(to_f64(q[i]), K, V, SM_SCALE)
                     for i, (K, V) in enumerate(_dequant_rows(rows, bt, bs, k_bs, v_bs))])
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_paged_prefill_equals_textbook_with_block_scales():
    """Each sequence's last min(3, L) tokens as causal queries: row j sees the
    positions up to its own, over rows dequantised with their blocks' scales."""
    G = 2
    q, rows, kc, vc, bt, ctx, k_bs, v_bs, Hkv, bs = _setup(G, seed=22)
    g = torch.Generator().manual_seed(5)
    nq = [min(3, int(L)) for L in ctx]
    qsl = torch.tensor([0] + list(np.cumsum(nq)), dtype=torch.int32)
    qp = torch.randn((int(qsl[-1]), Hkv * G, q.shape[2]), generator=g).to(torch.float16)
    got = oracle.paged_prefill(qp, kc, vc, bt, ctx, qsl, SM_SCALE, Hkv, k_bs, v_bs)
    deq = _dequant_rows(rows, bt, bs, k_bs, v_bs)
    for i, (K, V) in enumerate(deq):
        L = K.shape[0]
        for j in range(nq[i]):
            pos = L - nq[i] + j
            want = attention(to_f64(qp[int(qsl[i]) + j]), K[:pos + 1], V[:pos + 1], SM_SCALE)
            np.testing.assert_allclose(got[int(qsl[i]) + j], want, rtol=0, atol=1e-12)


def test_block_scales_equal_per_head_scales_when_blocks_agree_bitwise():
    q, rows, kc, vc, bt, ctx, _, _, Hkv, _ = _setup(2, seed=23)
    NB = kc.shape[0]
    kh = np.array([0.021, 0.0037, 0.11][:Hkv])
    vh = np.array([0.015, 0.0041, 0.093][:Hkv])
    per_head = oracle.paged_decode(q, kc, vc, bt, ctx, SM_SCALE, Hkv, kh, vh)
    per_block = oracle.paged_decode(q, kc, vc, bt, ctx, SM_SCALE, Hkv, np.tile(kh, (NB, 1)), np.tile(vh, (NB, 1)))
    assert np.array_equal(per_head, per_block)


def test_value_scale_of_one_block_enters_only_its_tokens():
    """Doubling the value scale of every block of one sequence's head doubles
    that head group's outputs exactly (a power of two) and leaves the other
    heads and the other sequences bit-identical; doubling a block no sequence
    reads changes nothing."""
    G = 2
    q, rows, kc, vc, bt, ctx, k_bs, v_bs, Hkv, bs = _setup(G, seed=24)
    base = oracle.paged_decode(q, kc, vc, bt, ctx, SM_SCALE, Hkv, k_bs, v_bs)
    s, h = 4, 1
    L = int(ctx[s])
    mine = sorted(set(bt[s, : -(-L // bs)].tolist()))
    v2 = v_bs.clone()
    v2[mine, h] *= 2.0
    got = oracle.paged_decode(q, kc, vc, bt, ctx, SM_SCALE, Hkv, k_bs, v2)
    grp = slice(h * G, (h + 1) * G)
    assert np.array_equal(got[s, grp], 2.0 * base[s, grp])
    mask = np.ones_like(got, dtype=bool)
    mask[s, grp] = False
    assert np.array_equal(got[mask], base[mask])
    used = set(bt[i, j].item() for i in range(len(rows)) for j in range(-(-int(ctx[i]) // bs)))
    spare = [b for b in range(kc.shape[0]) if b not in used]
    assert spare
    k3 = k_bs.clone()
    k3[spare[0]] *= 7.0
    assert np.array_equal(oracle.paged_decode(q, kc, vc, bt, ctx, SM_SCALE, Hkv, k3, v_bs), base)


def test_layers_take_their_own_block_scales():
    q, rows, kc, vc, bt, ctx, k_bs, v_bs, Hkv, _ = _setup(1, seed=25)
    k2, v2 = k_bs.flip(0), v_bs * 0.5
    got = oracle.paged_decode_layers(torch.stack([q, q]), torch.stack([kc, kc]), torch.stack([vc, vc]), bt, ctx,
                                     SM_SCALE, Hkv, torch.stack([k_bs, k2]), torch.stack([v_bs, v2]))
    assert np.array_equal(got[0], oracle.paged_decode(q, kc, vc, bt, ctx, SM_SCALE, Hkv, k_bs, v_bs))
    assert np.array_equal(got[1], oracle.paged_decode(q, kc, vc, bt, ctx, SM_SCALE, Hkv, k2, v2))


def test_cache_write_block_scales_match_torch_cast():
    """Each written row is torch's fp8 cast of x / (its destination block's
    scale for that head), the division in fp32, saturated at +-448 (the cast
    itself would give NaN past it); every other slot is untouched."""
    g = torch.Generator().manual_seed(26)
    NB, bs, Hkv, D = 4, 16, 3, 32
    kc = torch.zeros((NB, bs, Hkv, D), dtype=torch.uint8).view(torch.float8_e4m3fn)
    vc = kc.clone()
    k = (torch.randn((5, Hkv, D), generator=g) * 3.0).to(torch.bfloat16)
    v = (torch.randn((5, Hkv, D), generator=g) * 0.2).to(torch.float16)
    k_bs = (torch.rand((NB, Hkv), generator=g) * 0.05 + 0.001).to(torch.float32)
    v_bs = (torch.rand((NB, Hkv), generator=g) * 0.01 + 0.0002).to(torch.float32)
    slots = torch.tensor([0, 17, 47, 63, -1], dtype=torch.int64)
    nk, nv = oracle.cache_write(k, v.to(torch.bfloat16), kc, vc, slots, k_bs, v_bs)
    live = slots >= 0
    blk = slots[live] // bs
    ref_k = (k[live].float() / k_bs[blk][:, :, None]).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    ref_v = (v.to(torch.bfloat16)[live].float() / v_bs[blk][:, :, None]).clamp(-448, 448).to(
        torch.float8_e4m3fn).view(torch.uint8)
    assert (ref_k == 0x7E).any() or (ref_k == 0xFE).any()  # some rows saturate
    flat_k = nk.view(torch.uint8).view(NB * bs, Hkv, D)
    flat_v = nv.view(torch.uint8).view(NB * bs, Hkv, D)
    assert torch.equal(flat_k[slots[live]], ref_k)
    assert torch.equal(flat_v[slots[live]], ref_v)
    others = torch.ones(NB * bs, dtype=torch.bool)
    others[slots[live]] = False
    assert (flat_k[others] == 0).all() and (flat_v[others] == 0).all()


def test_block_scales_of_the_wrong_shape_are_refused():
    q, rows, kc, vc, bt, ctx, k_bs, v_bs, Hkv, _ = _setup(1, seed=27)
    with pytest.raises(ValueError):
        oracle.paged_decode(q, kc, vc, bt, ctx, SM_SCALE, Hkv, k_bs[:-1], v_bs[:-1])  # not [num_blocks, Hkv]

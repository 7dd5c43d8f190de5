"""Pins of the oracle's per-kv-head fp8 scales (one scale per kv head instead
of one per tensor: the precision chosen per attention head of section 8.2 of
page "vLLM框架中的KV cache优化与PagedAttention机制详解", applied to the fp8 KV
cache of page "大模型推理KV Cache内存管理与PagedAttention分页显存实战").

Each check rests on something other than the oracle itself: torch's own fp8
casts with numpy/scipy attention, the already-pinned per-tensor oracle, or an
exact power-of-two identity.  The heads get distinct scales throughout, so
reading the scale of the wrong head (query head instead of kv head, K's for
V's) fails at least one of them.
"""

import numpy as np
import pytest
import torch

import oracle
from tests.test_oracle import paginate
from tests.textbook import attention, to_f64

SM_SCALE = 0.125


def _fp8_rows(g, lens, Hkv, D, k_sc, v_sc, std):
    """Per-sequence (K, V) fp8 rows: kv head h holds N(0, std[h]^2) values
    encoded with its own scale (torch's cast, saturated to +-448)."""
    rows = []
    for L in lens:
        K = torch.randn((L, Hkv, D), generator=g) * std[None, :, None]
        V = torch.randn((L, Hkv, D), generator=g) * std[None, :, None]
        rows.append(((K / k_sc[None, :, None]).clamp(-448, 448).to(torch.float8_e4m3fn),
                     (V / v_sc[None, :, None]).clamp(-448, 448).to(torch.float8_e4m3fn)))
    return rows


def _setup(G, seed=7, lens=(1, 15, 16, 17, 50, 97), Hkv=4, D=64, bs=16):
    g = torch.Generator().manual_seed(seed)
    std = torch.tensor([0.25, 1.0, 4.0, 0.5][:Hkv], dtype=torch.float32)
    k_sc = (std * 4.5 / 448.0).to(torch.float32) * torch.tensor([1.0, 1.25, 0.875, 1.5][:Hkv])
    v_sc = (std * 4.5 / 448.0).to(torch.float32) * torch.tensor([1.5, 0.75, 1.125, 1.0][:Hkv])
    rows = _fp8_rows(g, lens, Hkv, D, k_sc, v_sc, std)
    q = torch.randn((len(lens), Hkv * G, D), generator=g).to(torch.float16)
    nb = sum(-(-L // bs) for L in lens) + 1
    kc, vc, bt, ctx = paginate(rows, bs, nb, "fp8")
    return q, rows, kc, vc, bt, ctx, k_sc, v_sc, Hkv


@pytest.mark.parametrize("G", [1, 4])
def test_identity_table_equals_textbook_with_head_scales(G):
    """Identity tables: paged decode equals contiguous attention over K, V
    decoded by torch's own fp8 cast, each kv head times its own scale."""
    q, rows, kc, vc, bt, ctx, k_sc, v_sc, Hkv = _setup(G)
    got = oracle.paged_decode(q, kc, vc, bt, ctx, SM_SCALE, Hkv, k_sc, v_sc)
    ks = k_sc.double().numpy()[None, :, None]
    vs = v_sc.double().numpy()[None, :, None]
    want = np.stack([attention(to_f64(q[i]), to_f64(K) * ks, to_f64(V) * vs, SM_SCALE)
                     for i, (K, V) in enumerate(rows)])
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_equal_head_scales_are_the_tensor_scale_bitwise():
    q, rows, kc, vc, bt, ctx, _, _, Hkv = _setup(2, seed=8)
    ks, vs = 0.0213, 0.0377
    per_tensor = oracle.paged_decode(q, kc, vc, bt, ctx, SM_SCALE, Hkv, ks, vs)
    per_head = oracle.paged_decode(q, kc, vc, bt, ctx, SM_SCALE, Hkv, np.full(Hkv, ks), np.full(Hkv, vs))
    assert np.array_equal(per_tensor, per_head)


def test_value_scale_of_one_head_scales_its_group_exactly():
    """Doubling kv head h's value scale doubles the outputs of its G query heads
    (exact: a power of two) and leaves every other head bit-identical."""
    G = 2
    q, rows, kc, vc, bt, ctx, k_sc, v_sc, Hkv = _setup(G, seed=9)
    base = oracle.paged_decode(q, kc, vc, bt, ctx, SM_SCALE, Hkv, k_sc, v_sc)
    for h in range(Hkv):
        v2 = v_sc.clone()
        v2[h] *= 2.0
        got = oracle.paged_decode(q, kc, vc, bt, ctx, SM_SCALE, Hkv, k_sc, v2)
        mine = slice(h * G, (h + 1) * G)
        assert np.array_equal(got[:, mine], 2.0 * base[:, mine])
        others = np.ones(Hkv * G, dtype=bool)
        others[mine] = False
        assert np.array_equal(got[:, others], base[:, others])


def test_key_scale_of_one_head_is_a_softmax_temperature():
    """Scaling kv head h's key scale by c equals the per-tensor oracle with
    softmax scale * c on that head's query group (the scores are scale q.(c K))."""
    G = 4
    q, rows, kc, vc, bt, ctx, _, _, Hkv = _setup(G, seed=10)
    ks, vs = 0.02, 0.03
    for h, c in [(0, 0.5), (1, 3.0), (3, 1.75)]:
        kh = np.full(Hkv, ks)
        kh[h] *= c
        got = oracle.paged_decode(q, kc, vc, bt, ctx, SM_SCALE, Hkv, kh, np.full(Hkv, vs))
        hot = oracle.paged_decode(q, kc, vc, bt, ctx, SM_SCALE * c, Hkv, ks, vs)
        cold = oracle.paged_decode(q, kc, vc, bt, ctx, SM_SCALE, Hkv, ks, vs)
        mine = slice(h * G, (h + 1) * G)
        np.testing.assert_allclose(got[:, mine], hot[:, mine], rtol=0, atol=1e-12)
        others = np.ones(Hkv * G, dtype=bool)
        others[mine] = False
        assert np.array_equal(got[:, others], cold[:, others])


def test_layers_take_their_own_row_of_head_scales():
    q, rows, kc, vc, bt, ctx, k_sc, v_sc, Hkv = _setup(1, seed=11)
    k2, v2 = k_sc.flip(0), v_sc * 0.5
    L_k = torch.stack([k_sc, k2])
    L_v = torch.stack([v_sc, v2])
    got = oracle.paged_decode_layers(torch.stack([q, q]), torch.stack([kc, kc]), torch.stack([vc, vc]), bt, ctx,
                                     SM_SCALE, Hkv, L_k, L_v)
    assert np.array_equal(got[0], oracle.paged_decode(q, kc, vc, bt, ctx, SM_SCALE, Hkv, k_sc, v_sc))
    assert np.array_equal(got[1], oracle.paged_decode(q, kc, vc, bt, ctx, SM_SCALE, Hkv, k2, v2))


def test_cache_write_head_scales_match_torch_cast():
    """Each head's row is encoded as torch's fp8 cast of x / (its head's scale),
    the division in fp32; every other slot is untouched."""
    g = torch.Generator().manual_seed(12)
    NB, bs, Hkv, D = 3, 16, 4, 64
    kc = torch.zeros((NB, bs, Hkv, D), dtype=torch.uint8).view(torch.float8_e4m3fn)
    vc = kc.clone()
    std = torch.tensor([0.25, 1.0, 4.0, 0.5])
    k = (torch.randn((3, Hkv, D), generator=g) * std[None, :, None]).to(torch.bfloat16)
    v = (torch.randn((3, Hkv, D), generator=g) * std[None, :, None]).to(torch.bfloat16)
    ks = torch.tensor([0.0031, 0.0117, 0.047, 0.0062], dtype=torch.float32)
    vs = torch.tensor([0.0029, 0.0125, 0.052, 0.0071], dtype=torch.float32)
    slots = torch.tensor([0, 17, 47], dtype=torch.int64)
    nk, nv = oracle.cache_write(k, v, kc, vc, slots, ks, vs)
    ref_k = (k.float() / ks[None, :, None]).to(torch.float8_e4m3fn).view(torch.uint8)
    ref_v = (v.float() / vs[None, :, None]).to(torch.float8_e4m3fn).view(torch.uint8)
    flat_k = nk.view(torch.uint8).view(NB * bs, Hkv, D)
    flat_v = nv.view(torch.uint8).view(NB * bs, Hkv, D)
    assert torch.equal(flat_k[slots], ref_k)
    assert torch.equal(flat_v[slots], ref_v)
    others = torch.ones(NB * bs, dtype=torch.bool)
    others[slots] = False
    assert (flat_k[others] == 0).all() and (flat_v[others] == 0).all()


def test_head_scale_errors():
    q, rows, kc, vc, bt, ctx, k_sc, v_sc, Hkv = _setup(1, seed=13)
    with pytest.raises(ValueError):  # one scale short
        oracle.paged_decode(q, kc, vc, bt, ctx, SM_SCALE, Hkv, k_sc[:-1], v_sc[:-1])
    k = torch.zeros((1, Hkv, 64), dtype=torch.float16)
    with pytest.raises(ValueError):
        oracle.cache_write(k, k, kc, vc, torch.tensor([0]), k_sc, v_sc[:2])


def _prefill_setup(G, seed):
    q_unused, rows, kc, vc, bt, ctx, k_sc, v_sc, Hkv = _setup(G, seed=seed)
    g = torch.Generator().manual_seed(seed + 100)
    lens = [int(x) for x in ctx]
    n = [min(L, r) for L, r in zip(lens, (1, 5, 16, 3, 20, 40))]
    qsl = torch.tensor([0] + list(np.cumsum(n)), dtype=torch.int32)
    q = torch.randn((int(qsl[-1]), Hkv * G, 64), generator=g).to(torch.float16)
    return q, rows, kc, vc, bt, ctx, qsl, n, k_sc, v_sc, Hkv


@pytest.mark.parametrize("G", [1, 4])
def test_prefill_with_head_scales_is_textbook_causal_attention(G):
    """Identity tables: query row j of a sequence with n rows and context L
    attends to positions 0 .. L - n + j of K, V decoded by torch's fp8 cast,
    each kv head times its own scale."""
    q, rows, kc, vc, bt, ctx, qsl, n, k_sc, v_sc, Hkv = _prefill_setup(G, 21)
    got = oracle.paged_prefill(q, kc, vc, bt, ctx, qsl, SM_SCALE, Hkv, k_sc, v_sc)
    ks = k_sc.double().numpy()[None, :, None]
    vs = v_sc.double().numpy()[None, :, None]
    for i, (K, V) in enumerate(rows):
        L = K.shape[0]
        for j in range(n[i]):
            r = int(qsl[i]) + j
            p = L - n[i] + j
            want = attention(to_f64(q[r]), to_f64(K[: p + 1]) * ks, to_f64(V[: p + 1]) * vs, SM_SCALE)
            np.testing.assert_allclose(got[r], want, rtol=0, atol=1e-12)


def test_prefill_rows_are_head_scaled_decodes_bitwise():
    """Each prefill row equals the per-head decode oracle over the context cut
    after its position, bit for bit; equal per-head scales equal the
    per-tensor prefill bit for bit."""
    q, rows, kc, vc, bt, ctx, qsl, n, k_sc, v_sc, Hkv = _prefill_setup(2, 22)
    got = oracle.paged_prefill(q, kc, vc, bt, ctx, qsl, SM_SCALE, Hkv, k_sc, v_sc)
    for i in range(len(n)):
        for j in range(n[i]):
            r = int(qsl[i]) + j
            cut = torch.tensor([int(ctx[i]) - n[i] + j + 1], dtype=torch.int32)
            dec = oracle.paged_decode(q[r:r + 1], kc, vc, bt[i:i + 1], cut, SM_SCALE, Hkv, k_sc, v_sc)
            assert np.array_equal(got[r], dec[0])
    ks, vs = 0.0213, 0.0377
    a = oracle.paged_prefill(q, kc, vc, bt, ctx, qsl, SM_SCALE, Hkv, ks, vs)
    b = oracle.paged_prefill(q, kc, vc, bt, ctx, qsl, SM_SCALE, Hkv, np.full(Hkv, ks), np.full(Hkv, vs))
    assert np.array_equal(a, b)

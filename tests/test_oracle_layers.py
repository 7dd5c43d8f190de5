"""Pins of the multi-layer decode oracle: each layer against textbook attention
over that layer's own rows through the shared tables, and the layer index
carried through (permuting layers permutes the result, bit for bit)."""

import numpy as np
import pytest
import torch

import oracle
from tests.test_oracle import paginate, rand_stored
from tests.textbook import attention, to_f64


def make_layers(seed, L, lens, Hkv, G, D, bs, dtype, order):
    g = torch.Generator().manual_seed(seed)
    nb = sum(-(-n // bs) for n in lens) + 1
    kcs, vcs, rows_all, bt, ctx = [], [], [], None, None
    for _ in range(L):
        rows = [(rand_stored(g, (n, Hkv, D), dtype), rand_stored(g, (n, Hkv, D), dtype)) for n in lens]
        kc, vc, bt, ctx = paginate(rows, bs, nb, dtype, order=order)  # the same placement in every layer
        kcs.append(kc)
        vcs.append(vc)
        rows_all.append(rows)
    qdt = "f16" if dtype == "fp8" else dtype
    q = rand_stored(g, (L, len(lens), Hkv * G, D), qdt)
    return q, torch.stack(kcs), torch.stack(vcs), bt, ctx, rows_all


@pytest.mark.parametrize("dtype,G", [("f32", 1), ("bf16", 4), ("f16", 2)])
def test_each_layer_is_textbook_attention_over_its_rows(dtype, G):
    lens, Hkv, D, bs, L = [1, 17, 40], 2, 32, 16, 3
    order = np.random.default_rng(7).permutation(sum(-(-n // bs) for n in lens) + 1)
    q, kc, vc, bt, ctx, rows = make_layers(10, L, lens, Hkv, G, D, bs, dtype, order)
    got = oracle.paged_decode_layers(q, kc, vc, bt, ctx, 0.15, Hkv)
    assert got.shape == (L, len(lens), Hkv * G, D)
    for layer in range(L):
        for i, (K, V) in enumerate(rows[layer]):
            want = attention(to_f64(q[layer, i]), to_f64(K), to_f64(V), 0.15)
            np.testing.assert_allclose(got[layer, i], want, rtol=0, atol=1e-12)


def test_permuting_layers_permutes_the_result_bitwise():
    lens, Hkv, G, D, bs, L = [5, 33, 64], 2, 4, 64, 16, 4
    q, kc, vc, bt, ctx, _ = make_layers(11, L, lens, Hkv, G, D, bs, "f16", None)
    a = oracle.paged_decode_layers(q, kc, vc, bt, ctx, 0.1, Hkv)
    perm = [2, 0, 3, 1]
    b = oracle.paged_decode_layers(q[perm], kc[perm], vc[perm], bt, ctx, 0.1, Hkv, nthreads=3)
    np.testing.assert_array_equal(b, a[perm])
    # layers are independent: a layer's result does not depend on the others
    np.testing.assert_array_equal(oracle.paged_decode_layers(q[1:2], kc[1:2], vc[1:2], bt, ctx, 0.1, Hkv)[0], a[1])


def test_layer_count_mismatch_is_an_error():
    lens, Hkv, G, D, bs, L = [5], 1, 1, 8, 16, 2
    q, kc, vc, bt, ctx, _ = make_layers(12, L, lens, Hkv, G, D, bs, "f32", None)
    with pytest.raises(ValueError):
        oracle.paged_decode_layers(q, kc[:1], vc, bt, ctx, 0.1, Hkv)

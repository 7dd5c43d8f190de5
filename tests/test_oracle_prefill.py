"""Pins of the prefill oracle (several causal query tokens per sequence).

As for decode, nothing here compares the oracle with itself re-typed: the
checks are textbook attention in numpy/scipy over each token's visible
prefix, torch's own causal scaled-dot-product attention, brute force on tiny
contexts, the (separately pinned) decode oracle on truncated contexts, and the
invariance of the result under physical block placement.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from tests.test_oracle import paginate, rand_stored
from tests.textbook import attention, to_f64


def causal_textbook(q, rows, qsl, scale, k_scale=1.0, v_scale=1.0):
    """Each query row of sequence i: textbook attention over the positions up to its own."""
    out = []
    for i, (K, V) in enumerate(rows):
        L = K.shape[0]
        nq = int(qsl[i + 1] - qsl[i])
        for j in range(nq):
            pos = L - nq + j
            out.append(attention(to_f64(q[int(qsl[i]) + j]), to_f64(K[: pos + 1]) * k_scale,
                                 to_f64(V[: pos + 1]) * v_scale, scale))
    return np.stack(out)


def make_case(seed, lens, q_lens, Hkv, G, D, bs, dtype, ks=1.0, vs=1.0):
    g = torch.Generator().manual_seed(seed)
    rows = [(rand_stored(g, (L, Hkv, D), dtype, ks), rand_stored(g, (L, Hkv, D), dtype, vs)) for L in lens]
    qsl = torch.tensor([0] + list(np.cumsum(q_lens)), dtype=torch.int32)
    qdt = "f16" if dtype == "fp8" else dtype
    q = rand_stored(g, (int(qsl[-1]), Hkv * G, D), qdt)
    return rows, qsl, q


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "fp8"])
@pytest.mark.parametrize("G", [1, 4])
def test_prefill_identity_table_equals_causal_textbook(dtype, G):
    Hkv, D, bs = 2, 64, 16
    lens, q_lens = [1, 16, 17, 50, 33], [1, 5, 17, 20, 0]
    ks, vs = (0.02, 0.03) if dtype == "fp8" else (1.0, 1.0)
    rows, qsl, q = make_case(200 + G, lens, q_lens, Hkv, G, D, bs, dtype, ks, vs)
    nb = sum(-(-L // bs) for L in lens) + 1
    kc, vc, bt, ctx = paginate(rows, bs, nb, dtype)
    got = oracle.paged_prefill(q, kc, vc, bt, ctx, qsl, 0.125, Hkv, ks, vs)
    want = causal_textbook(q, rows, qsl, 0.125, ks, vs)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("G", [1, 2])
def test_prefill_whole_prompt_equals_torch_causal_sdpa(G):
    """q_len = context: the whole prompt, against torch's causal attention (fp64, CPU)."""
    Hkv, D, bs = 2, 32, 16
    lens = [9, 40]
    rows, qsl, q = make_case(300 + G, lens, lens, Hkv, G, D, bs, "f32")
    kc, vc, bt, ctx = paginate(rows, bs, 8, "f32")
    got = oracle.paged_prefill(q, kc, vc, bt, ctx, qsl, 0.2, Hkv)
    for i, (K, V) in enumerate(rows):
        Qi = q[int(qsl[i]): int(qsl[i + 1])].double().transpose(0, 1)  # [H, L, D]
        Ki = K.double().repeat_interleave(G, dim=1).transpose(0, 1).contiguous()
        Vi = V.double().repeat_interleave(G, dim=1).transpose(0, 1).contiguous()
        ref = torch.nn.functional.scaled_dot_product_attention(Qi, Ki, Vi, is_causal=True, scale=0.2)
        np.testing.assert_allclose(got[int(qsl[i]): int(qsl[i + 1])], ref.transpose(0, 1).numpy(), rtol=0,
                                   atol=1e-12)


def test_prefill_rows_equal_decode_of_truncated_contexts():
    """Query token j of a sequence is a decode over the context cut after its own
    position (the decode oracle is pinned on its own)."""
    Hkv, G, D, bs = 2, 4, 64, 16
    lens, q_lens = [7, 48, 70], [7, 19, 33]
    rows, qsl, q = make_case(400, lens, q_lens, Hkv, G, D, bs, "bf16")
    kc, vc, bt, ctx = paginate(rows, bs, 12, "bf16", order=np.random.default_rng(4).permutation(12))
    got = oracle.paged_prefill(q, kc, vc, bt, ctx, qsl, 0.1, Hkv)
    for i, L in enumerate(lens):
        nq = q_lens[i]
        for j in range(nq):
            r = int(qsl[i]) + j
            cut = ctx.clone()
            cut[:] = 1
            cut[i] = L - nq + j + 1
            want = oracle.paged_decode(q[r: r + 1].repeat(len(lens), 1, 1), kc, vc, bt, cut, 0.1, Hkv)[i]
            np.testing.assert_array_equal(got[r], want)


def test_prefill_block_permutation_invariance_bitwise():
    Hkv, G, D, bs = 2, 2, 64, 16
    lens, q_lens = [30, 64, 81], [30, 10, 16]
    rows, qsl, q = make_case(500, lens, q_lens, Hkv, G, D, bs, "f16")
    kc, vc, bt, ctx = paginate(rows, bs, 16, "f16")
    a = oracle.paged_prefill(q, kc, vc, bt, ctx, qsl, 0.1, Hkv)
    kc2, vc2, bt2, ctx2 = paginate(rows, bs, 16, "f16", order=np.random.default_rng(11).permutation(16))
    assert not torch.equal(bt, bt2)
    b = oracle.paged_prefill(q, kc2, vc2, bt2, ctx2, qsl, 0.1, Hkv, nthreads=3)
    np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("L", [1, 2, 3])
def test_prefill_bruteforce_tiny(L):
    """Every q_len of a 1-3 token context, by explicit enumeration in plain Python."""
    Hkv, G, D, bs = 1, 2, 8, 16
    for nq in range(1, L + 1):
        rows, qsl, q = make_case(600 + 10 * L + nq, [L], [nq], Hkv, G, D, bs, "f32")
        kc, vc, bt, ctx = paginate(rows, bs, 2, "f32")
        got = oracle.paged_prefill(q, kc, vc, bt, ctx, qsl, 0.3, Hkv)
        K, V = rows[0][0].double().tolist(), rows[0][1].double().tolist()
        for j in range(nq):
            pos = L - nq + j
            for h in range(G):
                qv = q[j, h].double().tolist()
                s = [0.3 * sum(qv[d] * K[t][0][d] for d in range(D)) for t in range(pos + 1)]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                for d in range(D):
                    want = sum(e[t] * V[t][0][d] for t in range(pos + 1)) / sum(e)
                    assert abs(got[j, h, d] - want) < 1e-13


def test_prefill_errors():
    Hkv, G, D, bs = 1, 1, 8, 16
    rows, qsl, q = make_case(700, [4], [4], Hkv, G, D, bs, "f32")
    kc, vc, bt, ctx = paginate(rows, bs, 2, "f32")
    with pytest.raises(oracle.OracleError):  # more query tokens than the context holds
        oracle.paged_prefill(q, kc, vc, bt, ctx - 1, qsl, 0.3, Hkv)
    with pytest.raises(ValueError):  # query_start_loc must end at the row count
        oracle.paged_prefill(q, kc, vc, bt, ctx, torch.tensor([0, 3], dtype=torch.int32), 0.3, Hkv)

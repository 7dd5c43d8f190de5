"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Nothing here compares the oracle with itself re-typed: each check is a
library routine (torch / numpy dtype casts, scipy softmax), a closed form, an
invariant the pages imply, or brute force on tiny inputs.
"""

import math
import os

import numpy as np
import pytest
import torch

import oracle
from tests.textbook import attention, to_f64

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}


# --------------------------------------------------------------------------------------
# helpers: build a paged pool from contiguous per-sequence rows


def nan_like_pool(shape, dtype):
    if dtype == "fp8":
        return torch.full(shape, 0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn)
    return torch.full(shape, float("nan"), dtype=DT[dtype])


def paginate(rows, bs, num_blocks, dtype, order=None, width=None, trap=None):
    """rows: list of (K [L,Hkv,D], V [L,Hkv,D]) stored tensors.  Blocks are handed out
    in ``order`` (a sequence of physical ids); unused slots and padding are NaN."""
    Hkv, D = rows[0][0].shape[1:]
    kc = nan_like_pool((num_blocks, bs, Hkv, D), dtype)
    vc = nan_like_pool((num_blocks, bs, Hkv, D), dtype)
    order = list(range(num_blocks)) if order is None else list(order)
    need = [-(-K.shape[0] // bs) for K, _ in rows]
    width = width or max(need + [1])
    used = sum(need)
    trap = order[used] if trap is None else trap
    bt = torch.full((len(rows), width), trap, dtype=torch.int32)
    nxt = 0
    kb, vb = kc.view(torch.uint8) if dtype == "fp8" else kc, vc.view(torch.uint8) if dtype == "fp8" else vc
    for i, (K, V) in enumerate(rows):
        Kb = K.view(torch.uint8) if dtype == "fp8" else K
        Vb = V.view(torch.uint8) if dtype == "fp8" else V
        for j in range(need[i]):
            b = order[nxt]
            nxt += 1
            bt[i, j] = b
            lo, hi = j * bs, min(K.shape[0], (j + 1) * bs)
            kb[b, : hi - lo] = Kb[lo:hi]
            vb[b, : hi - lo] = Vb[lo:hi]
    ctx = torch.tensor([K.shape[0] for K, _ in rows], dtype=torch.int32)
    return kc, vc, bt, ctx


def rand_stored(gen, shape, dtype, scale=1.0):
    x = torch.randn(shape, generator=gen, dtype=torch.float32)
    if dtype == "fp8":
        return (x / scale).to(torch.float8_e4m3fn)
    return x.to(DT[dtype])


def textbook_for(q, rows, scale, k_scale=1.0, v_scale=1.0):
    out = []
    for i, (K, V) in enumerate(rows):
        out.append(attention(to_f64(q[i]), to_f64(K) * k_scale, to_f64(V) * v_scale, scale))
    return np.stack(out)


# --------------------------------------------------------------------------------------
# exact decoders: every code against torch / numpy's own casts


def test_f16_decoder_exhaustive():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_double(int(b)) for b in bits])
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])


def test_bf16_decoder_exhaustive():
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    ref = bits.view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.bf16_to_double(int(b) & 0xFFFF) for b in bits.tolist()])
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])


def test_fp8_decoder_exhaustive():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.fp8_to_double(c) for c in range(256)])
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    assert np.isnan(got).sum() == 2  # S.1111.111 only
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])


def test_fp8_spec_points():
    """Landmark values of the OCP 8-bit e4m3 format (tests/golden/e4m3fn_spec_points.txt)."""
    n = 0
    with open(os.path.join(GOLDEN, "e4m3fn_spec_points.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            code, value = line.split()
            code = int(code, 16)
            v = oracle.fp8_to_double(code)
            if value == "nan":
                assert math.isnan(v)
            else:
                assert v == float.fromhex(value) if value.startswith(("0x", "-0x")) else v == float(value)
            n += 1
    assert n >= 8


def test_fp8_encoder_roundtrip_and_ties():
    finite = [c for c in range(256) if (c & 0x7F) != 0x7F]
    for c in finite:
        assert oracle.float_to_fp8(oracle.fp8_to_double(c)) == c
    # midpoints between neighbouring non-negative codes go to the even code
    for c in range(0, 0x7E):
        lo, hi = oracle.fp8_to_double(c), oracle.fp8_to_double(c + 1)
        mid = np.float32((lo + hi) / 2)
        assert float(mid) == (lo + hi) / 2  # midpoints are exact in fp32
        want = c if c % 2 == 0 else c + 1
        assert oracle.float_to_fp8(float(mid)) == want
        assert oracle.float_to_fp8(-float(mid)) == want | 0x80


def test_fp8_encoder_matches_torch_in_range():
    g = torch.Generator().manual_seed(11)
    x = torch.cat([
        torch.randn(20000, generator=g) * 30,
        torch.randn(20000, generator=g) * 0.01,
        (torch.rand(5000, generator=g) * 2 - 1) * 464,
    ]).to(torch.float32)
    ref = x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.float_to_fp8(float(v)) for v in x.tolist()], dtype=np.uint8)
    np.testing.assert_array_equal(got, ref)


def test_fp8_encoder_saturates():
    for x, code in [(448.0, 0x7E), (449.0, 0x7E), (480.0, 0x7E), (1e6, 0x7E), (float("inf"), 0x7E),
                    (-500.0, 0xFE), (float("-inf"), 0xFE)]:
        assert oracle.float_to_fp8(x) == code
    assert oracle.float_to_fp8(float("nan")) & 0x7F == 0x7F


# --------------------------------------------------------------------------------------
# attention values


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "fp8"])
@pytest.mark.parametrize("G", [1, 4])
def test_identity_table_equals_textbook(dtype, G):
    g = torch.Generator().manual_seed(100 + G)
    Hkv, D, bs = 2, 64, 16
    H = Hkv * G
    lens = [1, 15, 16, 17, 50]
    ks, vs = (0.02, 0.03) if dtype == "fp8" else (1.0, 1.0)
    rows = [(rand_stored(g, (L, Hkv, D), dtype, ks), rand_stored(g, (L, Hkv, D), dtype, vs)) for L in lens]
    qdt = "f16" if dtype == "fp8" else dtype
    q = rand_stored(g, (len(lens), H, D), qdt)
    nb = sum(-(-L // bs) for L in lens) + 1
    kc, vc, bt, ctx = paginate(rows, bs, nb, dtype)  # identity placement, in order
    got = oracle.paged_decode(q, kc, vc, bt, ctx, 0.125, Hkv, ks, vs)
    want = textbook_for(q, rows, 0.125, ks, vs)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_block_permutation_invariance_bitwise():
    g = torch.Generator().manual_seed(5)
    Hkv, D, bs, H = 4, 64, 16, 4
    lens = [3, 40, 64, 81]
    rows = [(rand_stored(g, (L, Hkv, D), "f16"), rand_stored(g, (L, Hkv, D), "f16")) for L in lens]
    q = rand_stored(g, (4, H, D), "f16")
    nb = 40
    kc, vc, bt, ctx = paginate(rows, bs, nb, "f16")
    a = oracle.paged_decode(q, kc, vc, bt, ctx, 0.1, Hkv)
    order = np.random.default_rng(9).permutation(nb)
    kc2, vc2, bt2, ctx2 = paginate(rows, bs, nb, "f16", order=order)
    assert not torch.equal(bt, bt2)
    b = oracle.paged_decode(q, kc2, vc2, bt2, ctx2, 0.1, Hkv)
    np.testing.assert_array_equal(a, b)


def test_shared_prefix_equals_private_copies_bitwise():
    g = torch.Generator().manual_seed(6)
    Hkv, D, bs, H = 2, 64, 16, 2
    prefix_k = rand_stored(g, (32, Hkv, D), "bf16")
    prefix_v = rand_stored(g, (32, Hkv, D), "bf16")
    suffixes = [(rand_stored(g, (L, Hkv, D), "bf16"), rand_stored(g, (L, Hkv, D), "bf16")) for L in (1, 16, 23)]
    rows = [(torch.cat([prefix_k, sk]), torch.cat([prefix_v, sv])) for sk, sv in suffixes]
    q = rand_stored(g, (3, H, D), "bf16")
    # private copies
    kc, vc, bt, ctx = paginate(rows, bs, 20, "bf16")
    a = oracle.paged_decode(q, kc, vc, bt, ctx, 0.1, Hkv)
    # shared: the two prefix blocks of sequence 0 referenced by all three
    bt_s = bt.clone()
    for i in (1, 2):
        bt_s[i, :2] = bt[0, :2]
    # poison the now-unreferenced private prefix copies
    for i in (1, 2):
        for j in range(2):
            kc[bt[i, j]] = float("nan")
            vc[bt[i, j]] = float("nan")
    b = oracle.paged_decode(q, kc, vc, bt_s, ctx, 0.1, Hkv)
    np.testing.assert_array_equal(a, b)


def test_identical_keys_give_mean_of_v():
    g = torch.Generator().manual_seed(7)
    Hkv, D, bs, H = 2, 64, 16, 4
    L = 37
    krow = rand_stored(g, (1, Hkv, D), "f32")
    rows = [(krow.expand(L, Hkv, D).contiguous(), rand_stored(g, (L, Hkv, D), "f32"))]
    q = rand_stored(g, (1, H, D), "f32")
    kc, vc, bt, ctx = paginate(rows, bs, 4, "f32")
    got = oracle.paged_decode(q, kc, vc, bt, ctx, 0.3, Hkv)[0]
    V = to_f64(rows[0][1])
    for h in range(H):
        np.testing.assert_allclose(got[h], V[:, h // 2, :].mean(axis=0), rtol=0, atol=1e-14)


def test_ctx1_is_v0_exactly():
    g = torch.Generator().manual_seed(8)
    rows = [(rand_stored(g, (1, 2, 64), "f16"), rand_stored(g, (1, 2, 64), "f16"))]
    q = rand_stored(g, (1, 2, 64), "f16")
    kc, vc, bt, ctx = paginate(rows, 16, 3, "f16")
    got = oracle.paged_decode(q, kc, vc, bt, ctx, 0.125, 2)[0]
    np.testing.assert_array_equal(got, to_f64(rows[0][1])[0])


def test_ctx2_closed_form():
    g = torch.Generator().manual_seed(9)
    rows = [(rand_stored(g, (2, 1, 64), "f32"), rand_stored(g, (2, 1, 64), "f32"))]
    q = rand_stored(g, (1, 1, 64), "f32")
    kc, vc, bt, ctx = paginate(rows, 16, 3, "f32")
    got = oracle.paged_decode(q, kc, vc, bt, ctx, 0.2, 1)[0, 0]
    K, V, qq = to_f64(rows[0][0])[:, 0], to_f64(rows[0][1])[:, 0], to_f64(q)[0, 0]
    s0, s1 = 0.2 * (qq @ K[0]), 0.2 * (qq @ K[1])
    w0 = 1.0 / (1.0 + math.exp(s1 - s0))
    np.testing.assert_allclose(got, w0 * V[0] + (1 - w0) * V[1], rtol=0, atol=1e-14)


@pytest.mark.parametrize("L", [1, 2, 3])
def test_bruteforce_tiny_contexts(L):
    """Pure-Python loops over the stored values, token by token, block by block."""
    g = torch.Generator().manual_seed(20 + L)
    Hkv, D, bs, H = 1, 4, 2, 2
    rows = [(rand_stored(g, (L, Hkv, D), "f32"), rand_stored(g, (L, Hkv, D), "f32"))]
    q = rand_stored(g, (1, H, D), "f32")
    order = [3, 0, 2, 1]
    kc, vc, bt, ctx = paginate(rows, bs, 4, "f32", order=order)
    got = oracle.paged_decode(q, kc, vc, bt, ctx, 0.7, Hkv)[0]
    Kl = rows[0][0].tolist()
    Vl = rows[0][1].tolist()
    ql = q.tolist()[0]
    for h in range(H):
        s = [0.7 * sum(ql[h][d] * Kl[t][0][d] for d in range(D)) for t in range(L)]
        e = [math.exp(x - max(s)) for x in s]
        z = sum(e)
        want = [sum(e[t] * Vl[t][0][d] for t in range(L)) / z for d in range(D)]
        np.testing.assert_allclose(got[h], want, rtol=0, atol=1e-14)


def _grid_values(g, shape, step=2.0 ** -8):
    # N(0,1) rounded to multiples of 2^-8: exact in fp32 after shifts and affine maps
    return (torch.round(torch.randn(shape, generator=g) / step) * step).to(torch.float32)


def test_shift_invariance_large_offset():
    """Adding one vector u to every key shifts all scores by scale*q.u (here > 1000):
    the softmax is unchanged and must not overflow."""
    g = torch.Generator().manual_seed(10)
    Hkv, D, H, L = 1, 64, 1, 45
    K = _grid_values(g, (L, Hkv, D))
    V = _grid_values(g, (L, Hkv, D))
    q = _grid_values(g, (1, H, D))
    u = 512.0 * torch.sign(q[0, 0])
    scale = 0.125
    assert scale * float(q[0, 0] @ u) > 1000
    a = oracle.paged_decode(q, *paginate([(K, V)], 16, 4, "f32"), scale, Hkv)
    Ks = K + u  # exact in fp32
    b = oracle.paged_decode(q, *paginate([(Ks, V)], 16, 4, "f32"), scale, Hkv)
    assert np.isfinite(b).all()
    np.testing.assert_allclose(b, a, rtol=0, atol=1e-11)


def test_v_affine_map():
    g = torch.Generator().manual_seed(12)
    Hkv, D, H, L = 2, 64, 2, 70
    K = _grid_values(g, (L, Hkv, D))
    V = _grid_values(g, (L, Hkv, D))
    q = _grid_values(g, (1, H, D))
    alpha, beta = 2.0, 0.5
    pa = paginate([(K, V)], 16, 6, "f32")
    pb = paginate([(K, alpha * V + beta)], 16, 6, "f32")
    a = oracle.paged_decode(q, *pa, 0.1, Hkv)
    b = oracle.paged_decode(q, *pb, 0.1, Hkv)
    np.testing.assert_allclose(b, alpha * a + beta, rtol=0, atol=1e-12)


def test_gqa_equals_replicated_mha():
    g = torch.Generator().manual_seed(13)
    Hkv, G, D = 2, 4, 64
    H = Hkv * G
    lens = [5, 33]
    rows = [(rand_stored(g, (L, Hkv, D), "f16"), rand_stored(g, (L, Hkv, D), "f16")) for L in lens]
    q = rand_stored(g, (2, H, D), "f16")
    a = oracle.paged_decode(q, *paginate(rows, 16, 8, "f16"), 0.1, Hkv)
    rep = [(K.repeat_interleave(G, dim=1), V.repeat_interleave(G, dim=1)) for K, V in rows]
    b = oracle.paged_decode(q, *paginate(rep, 16, 8, "f16"), 0.1, H)
    np.testing.assert_array_equal(a, b)


def test_poison_in_unread_slots_never_reaches_output():
    g = torch.Generator().manual_seed(14)
    Hkv, D, H = 2, 64, 2
    lens = [7, 16, 30]
    rows = [(rand_stored(g, (L, Hkv, D), "f16"), rand_stored(g, (L, Hkv, D), "f16")) for L in lens]
    q = rand_stored(g, (3, H, D), "f16")
    kc, vc, bt, ctx = paginate(rows, 16, 9, "f16", width=6)  # NaN tails, NaN trap padding
    a = oracle.paged_decode(q, kc, vc, bt, ctx, 0.1, Hkv)
    assert np.isfinite(a).all()
    kz, vz = torch.nan_to_num(kc, nan=0.0), torch.nan_to_num(vc, nan=0.0)
    b = oracle.paged_decode(q, kz, vz, bt, ctx, 0.1, Hkv)
    np.testing.assert_array_equal(a, b)


def test_zero_context_gives_zeros():
    g = torch.Generator().manual_seed(15)
    rows = [(rand_stored(g, (3, 1, 64), "f32"), rand_stored(g, (3, 1, 64), "f32"))]
    q = rand_stored(g, (2, 1, 64), "f32")
    kc, vc, bt, _ = paginate(rows, 16, 2, "f32")
    bt = torch.cat([bt, bt])
    ctx = torch.tensor([3, 0], dtype=torch.int32)
    out = oracle.paged_decode(q, kc, vc, bt, ctx, 0.1, 1)
    assert (out[1] == 0).all() and np.isfinite(out[0]).all()


def test_thread_count_does_not_change_result():
    g = torch.Generator().manual_seed(16)
    lens = [100, 3, 64, 17, 250, 1]
    rows = [(rand_stored(g, (L, 2, 64), "bf16"), rand_stored(g, (L, 2, 64), "bf16")) for L in lens]
    q = rand_stored(g, (6, 8, 64), "bf16")
    p = paginate(rows, 16, 40, "bf16")
    a = oracle.paged_decode(q, *p, 0.1, 2, nthreads=1)
    b = oracle.paged_decode(q, *p, 0.1, 2, nthreads=5)
    np.testing.assert_array_equal(a, b)


def test_decode_errors():
    g = torch.Generator().manual_seed(17)
    rows = [(rand_stored(g, (20, 1, 64), "f32"), rand_stored(g, (20, 1, 64), "f32"))]
    q = rand_stored(g, (1, 1, 64), "f32")
    kc, vc, bt, ctx = paginate(rows, 16, 3, "f32")
    bad = bt.clone()
    bad[0, 1] = 99
    with pytest.raises(oracle.OracleError):
        oracle.paged_decode(q, kc, vc, bad, ctx, 0.1, 1)
    with pytest.raises(oracle.OracleError):
        oracle.paged_decode(q, kc, vc, bt, torch.tensor([33], dtype=torch.int32), 0.1, 1)


# --------------------------------------------------------------------------------------
# cache write


def test_cache_write_places_rows_and_touches_nothing_else():
    g = torch.Generator().manual_seed(18)
    NB, bs, Hkv, D = 6, 16, 2, 64
    kc = rand_stored(g, (NB, bs, Hkv, D), "bf16")
    vc = rand_stored(g, (NB, bs, Hkv, D), "bf16")
    k = rand_stored(g, (4, Hkv, D), "bf16")
    v = rand_stored(g, (4, Hkv, D), "bf16")
    slots = torch.tensor([5, -1, 95, 16], dtype=torch.int64)
    nk, nv = oracle.cache_write(k, v, kc, vc, slots)
    ek, ev = kc.clone().view(NB * bs, Hkv, D), vc.clone().view(NB * bs, Hkv, D)
    keep = slots >= 0
    ek[slots[keep]] = k[keep]
    ev[slots[keep]] = v[keep]
    assert torch.equal(nk.view(torch.int16), ek.view(NB, bs, Hkv, D).view(torch.int16))
    assert torch.equal(nv.view(torch.int16), ev.view(NB, bs, Hkv, D).view(torch.int16))


def test_cache_write_fp8_matches_torch_cast():
    g = torch.Generator().manual_seed(19)
    NB, bs, Hkv, D = 3, 16, 2, 64
    kc = torch.zeros((NB, bs, Hkv, D), dtype=torch.uint8).view(torch.float8_e4m3fn)
    vc = kc.clone()
    k = (torch.randn((3, Hkv, D), generator=g) * 3).to(torch.float16)
    v = (torch.randn((3, Hkv, D), generator=g) * 3).to(torch.float16)
    ks, vs = 0.0213, 0.0377
    slots = torch.tensor([0, 17, 47], dtype=torch.int64)
    nk, nv = oracle.cache_write(k, v, kc, vc, slots, ks, vs)
    ref_k = (k.float() / torch.tensor(ks, dtype=torch.float32)).to(torch.float8_e4m3fn).view(torch.uint8)
    ref_v = (v.float() / torch.tensor(vs, dtype=torch.float32)).to(torch.float8_e4m3fn).view(torch.uint8)
    flat_k = nk.view(torch.uint8).view(NB * bs, Hkv, D)
    flat_v = nv.view(torch.uint8).view(NB * bs, Hkv, D)
    assert torch.equal(flat_k[slots], ref_k)
    assert torch.equal(flat_v[slots], ref_v)
    others = torch.ones(NB * bs, dtype=torch.bool)
    others[slots] = False
    assert (flat_k[others] == 0).all() and (flat_v[others] == 0).all()


def test_cache_write_rejects_duplicates_and_out_of_pool():
    k = torch.zeros((2, 1, 64), dtype=torch.float32)
    kc = torch.zeros((2, 16, 1, 64), dtype=torch.float32)
    with pytest.raises(oracle.OracleError):
        oracle.cache_write(k, k, kc, kc, torch.tensor([3, 3]))
    with pytest.raises(oracle.OracleError):
        oracle.cache_write(k, k, kc, kc, torch.tensor([3, 32]))

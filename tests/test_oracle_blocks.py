"""Pins of the block-copy oracle (copy-on-write of a shared block, swap of
whole blocks between pools).

The checks are element-by-element brute force in plain Python, the untouched
rest of the pool, and what a copy must preserve on the pages' own terms: a
sequence that copies a shared, partly filled block before writing into it
sees textbook attention over its own tokens while the other sharer's result
stays bit-identical; blocks swapped out to a host pool and back into other
physical ids give the same decode, bit for bit.
"""

import numpy as np
import pytest
import torch

import oracle
from tests.test_oracle import DT, nan_like_pool, paginate, rand_stored
from tests.textbook import attention, to_f64


def _pool(g, nb, bs, Hkv, D, dtype):
    return rand_stored(g, (nb, bs, Hkv, D), dtype)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "fp8"])
def test_copy_blocks_bruteforce_elements(dtype):
    g = torch.Generator().manual_seed(1)
    nb, bs, Hkv, D = 9, 4, 2, 3
    src = _pool(g, nb, bs, Hkv, D, dtype)
    dst = _pool(g, 7, bs, Hkv, D, dtype)
    pairs = torch.tensor([[8, 0], [2, 5], [-1, 3], [2, 6], [4, -1]], dtype=torch.int64)
    got = oracle.copy_blocks(dst, src, pairs)
    sb = src.view(torch.uint8) if dtype == "fp8" else src
    db = dst.view(torch.uint8) if dtype == "fp8" else dst
    gb = got.view(torch.uint8) if dtype == "fp8" else got
    want_src = {0: 8, 5: 2, 6: 2}  # destination -> source; pairs with a negative id do nothing
    for b in range(7):
        for r in range(bs):
            for h in range(Hkv):
                for x in range(D):
                    ref = sb[want_src[b], r, h, x] if b in want_src else db[b, r, h, x]
                    a, e = gb[b, r, h, x].item(), ref.item()
                    assert a == e or (a != a and e != e), (b, r, h, x)
    # the caller's tensors are untouched unless asked
    assert not torch.equal(got.view(torch.uint8), dst.view(torch.uint8))


def test_copy_blocks_inplace_and_int32_mapping():
    g = torch.Generator().manual_seed(2)
    pool = _pool(g, 6, 16, 2, 8, "f16")
    before = pool.clone()
    out = oracle.copy_blocks(pool, pool, torch.tensor([[1, 4], [3, 5]], dtype=torch.int32), inplace=True)
    assert out is pool
    assert torch.equal(pool[4], before[1]) and torch.equal(pool[5], before[3])
    assert torch.equal(pool[:4], before[:4])


def test_copy_on_write_of_a_partly_filled_shared_block():
    """Two sequences share a 20-token prefix (blocks p0 full, p1 with 4 tokens).
    Sequence B appends a token: p1 is copied to a fresh block q first, B's table
    points at q, and the new token goes into q.  A's decode stays bit-identical;
    B's equals textbook attention over prefix + its token."""
    g = torch.Generator().manual_seed(3)
    bs, Hkv, G, D, nb = 16, 2, 2, 32, 8
    L = 20
    K = rand_stored(g, (L, Hkv, D), "bf16")
    V = rand_stored(g, (L, Hkv, D), "bf16")
    kc, vc, bt, ctx = paginate([(K, V)], bs, nb, "bf16")
    p0, p1 = int(bt[0, 0]), int(bt[0, 1])
    q = rand_stored(g, (2, Hkv * G, D), "bf16")
    tables = torch.tensor([[p0, p1], [p0, p1]], dtype=torch.int32)
    lens = torch.tensor([L, L], dtype=torch.int32)
    a_before = oracle.paged_decode(q, kc, vc, tables, lens, 0.2, Hkv)
    # copy-on-write for B, then the append
    fresh = 5
    kc = oracle.copy_blocks(kc, kc, torch.tensor([[p1, fresh]]))
    vc = oracle.copy_blocks(vc, vc, torch.tensor([[p1, fresh]]))
    tables[1, 1] = fresh
    kn = rand_stored(g, (1, Hkv, D), "bf16")
    vn = rand_stored(g, (1, Hkv, D), "bf16")
    kc, vc = oracle.cache_write(kn, vn, kc, vc, torch.tensor([fresh * bs + (L % bs)]))
    lens[1] = L + 1
    after = oracle.paged_decode(q, kc, vc, tables, lens, 0.2, Hkv)
    np.testing.assert_array_equal(after[0], a_before[0])
    want_b = attention(to_f64(q[1]), to_f64(torch.cat([K, kn])), to_f64(torch.cat([V, vn])), 0.2)
    np.testing.assert_allclose(after[1], want_b, rtol=0, atol=1e-12)
    # the shared block itself was not written
    assert torch.isnan(kc[p1, L % bs].float()).all()


@pytest.mark.parametrize("dtype", ["f16", "fp8"])
def test_swap_out_and_back_into_other_blocks_is_bitwise_neutral(dtype):
    g = torch.Generator().manual_seed(4)
    bs, Hkv, D, nb = 16, 2, 64, 24
    ks, vs = (0.02, 0.03) if dtype == "fp8" else (1.0, 1.0)
    rows = [(rand_stored(g, (L, Hkv, D), dtype, ks), rand_stored(g, (L, Hkv, D), dtype, vs)) for L in (40, 70)]
    kc, vc, bt, ctx = paginate(rows, bs, nb, dtype)
    q = rand_stored(g, (2, Hkv, D), "f16")
    ref = oracle.paged_decode(q, kc, vc, bt, ctx, 0.125, Hkv, ks, vs)
    used = sorted({int(b) for i in range(2) for b in bt[i, : -(-int(ctx[i]) // bs)]})
    host_k = nan_like_pool((len(used), bs, Hkv, D), dtype)
    host_v = nan_like_pool((len(used), bs, Hkv, D), dtype)
    out_map = torch.tensor([[b, i] for i, b in enumerate(used)])
    host_k = oracle.copy_blocks(host_k, kc, out_map)
    host_v = oracle.copy_blocks(host_v, vc, out_map)
    # the device pool is reused by others meanwhile; the blocks come back elsewhere
    kc2, vc2 = nan_like_pool(kc.shape, dtype), nan_like_pool(vc.shape, dtype)
    new_ids = list(range(nb - 1, nb - 1 - len(used), -1))
    in_map = torch.tensor([[i, new_ids[i]] for i in range(len(used))])
    kc2 = oracle.copy_blocks(kc2, host_k, in_map)
    vc2 = oracle.copy_blocks(vc2, host_v, in_map)
    remap = {b: new_ids[i] for i, b in enumerate(used)}
    bt2 = bt.clone()
    for i in range(2):
        for j in range(-(-int(ctx[i]) // bs)):
            bt2[i, j] = remap[int(bt[i, j])]
    got = oracle.paged_decode(q, kc2, vc2, bt2, ctx, 0.125, Hkv, ks, vs)
    np.testing.assert_array_equal(got, ref)


def test_copy_blocks_errors():
    g = torch.Generator().manual_seed(5)
    pool = _pool(g, 4, 16, 1, 8, "f32")
    other = _pool(g, 4, 16, 1, 8, "f32")
    with pytest.raises(oracle.OracleError):  # past the pool
        oracle.copy_blocks(other, pool, torch.tensor([[4, 0]]))
    with pytest.raises(oracle.OracleError):
        oracle.copy_blocks(other, pool, torch.tensor([[0, 4]]))
    with pytest.raises(oracle.OracleError):  # a destination twice
        oracle.copy_blocks(other, pool, torch.tensor([[0, 1], [2, 1]]))
    with pytest.raises(oracle.OracleError):  # same pool: destination is also a source
        oracle.copy_blocks(pool, pool, torch.tensor([[0, 1], [1, 2]]))
    # different pools: a destination id may equal a source id
    oracle.copy_blocks(other, pool, torch.tensor([[0, 1], [1, 2]]))
    with pytest.raises(ValueError):  # block shapes differ
        oracle.copy_blocks(_pool(g, 4, 16, 2, 8, "f32"), pool, torch.tensor([[0, 0]]))

"""GPU parity of fp8 caches with one scale per (physical block, kv head),
through the C ABI, against the fp64 oracle: the cache write (each new row
quantised with its destination block's scales; bit-exact over the whole pool),
single-layer decode on both kernels (vector ALU for groups of 1-2, matrix
cores for 4-16) across work splits, multi-layer decode with a slab of scales
per layer, and PA_FLAG_VALIDATE on the scales.  Prefill with per-block scales
is in tests/test_gpu_prefill.py (fp8_blocks_* cases)."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_447_amd as pa
from pa_workloads import get_config, scaled
from tests.gpu_common import (NTHREADS, TOL_F32, TOL_OUT, gpu_cache_write, gpu_decode, host_inputs, log,
                              max_abs_err, max_err_beyond_rounding, oracle_step, setup)

pytestmark = pytest.mark.gpu


def _bytes(t):
    return t.detach().cpu().contiguous().view(torch.uint8)


def _check_step(cfg, name, part=None, workers=0):
    layout, inp = setup(cfg)
    assert torch.is_tensor(inp["k_scale"]) and tuple(inp["k_scale"].shape) == (cfg.num_blocks, cfg.num_kv_heads)
    host = host_inputs(inp)
    gpu_cache_write(cfg, inp)
    ws = pa.new_workspace(inp["q"], cfg.num_kv_heads, workers)
    out = gpu_decode(cfg, inp, partition_size=part, num_workers=workers, workspace=ws)
    out32 = gpu_decode(cfg, inp, out_dtype=torch.float32, partition_size=part, num_workers=workers, workspace=ws)
    torch.cuda.synchronize()
    ref, kc, vc = oracle_step(cfg, host)
    assert torch.equal(_bytes(inp["k_cache"]), kc.view(torch.uint8)), "k_cache differs from the oracle's write"
    assert torch.equal(_bytes(inp["v_cache"]), vc.view(torch.uint8)), "v_cache differs from the oracle's write"
    err, err32 = max_abs_err(out, ref), max_abs_err(out32, ref)
    beyond = max_err_beyond_rounding(out, ref)
    log(f"[{name}] err={err:.3e} (beyond output rounding {beyond:.3e}) err32={err32:.3e} "
        f"max|ref|={np.abs(ref).max():.3f}")
    assert beyond <= TOL_OUT["fp8"]
    assert err32 <= TOL_F32["fp8"]
    return inp


def test_full_size_gqa70b_fp8_blocks_step_matches_oracle():
    cfg = get_config("gqa70b_fp8_blocks")
    log(f"[{cfg.name}] generating")
    _check_step(cfg, cfg.name)


_BASE = get_config("gqa70b_fp8_blocks")
SMALL = {
    "mha_f16q_bs16": scaled(_BASE, num_seqs=6, num_heads=8, num_kv_heads=8, block_size=16, num_blocks=1500,
                            max_blocks_per_seq=160, ctx_hi=2500, allocator="shuffled"),
    "gqa2_bf16q_d64": scaled(_BASE, num_seqs=7, num_heads=8, num_kv_heads=4, head_dim=64, q_dtype="bf16",
                             num_blocks=900, max_blocks_per_seq=80, ctx_hi=2500),
    "gqa4_f16q_d64_bs16": scaled(_BASE, num_seqs=5, num_heads=16, num_kv_heads=4, head_dim=64, block_size=16,
                                 num_blocks=1200, max_blocks_per_seq=128, ctx_hi=2000, allocator="shuffled"),
    "gqa8_f16q": scaled(_BASE, num_seqs=9, num_blocks=1500, max_blocks_per_seq=64, ctx_hi=2048),
    "gqa16_bf16q": scaled(_BASE, num_seqs=5, num_heads=32, num_kv_heads=2, q_dtype="bf16", num_blocks=700,
                          max_blocks_per_seq=64, ctx_hi=2048),
}
SPLITS = [(0, 0), (256, 0), (0, 7), (32, 65536)]


@pytest.mark.parametrize("case", sorted(SMALL))
@pytest.mark.parametrize("split", SPLITS, ids=[f"p{p}w{w}" for p, w in SPLITS])
def test_small_block_scale_cases_match_oracle(case, split):
    part, workers = split
    cfg = SMALL[case]
    _check_step(cfg, f"{case} p={part} w={workers}", part if part % cfg.block_size == 0 else 0, workers)


def test_layers_take_their_own_block_scales():
    """Two layers over the same pool with different block scales (the second
    reversed over the blocks and halved): each layer equals the oracle with its
    own slab of scales."""
    cfg = SMALL["gqa4_f16q_d64_bs16"]
    layout, inp = setup(cfg)
    gpu_cache_write(cfg, inp)
    torch.cuda.synchronize()
    ks1, vs1 = inp["k_scale"], inp["v_scale"]
    ks2, vs2 = ks1.flip(0).contiguous(), (vs1 * 0.5).contiguous()
    q2 = torch.stack([inp["q"], inp["q"].flip(0).contiguous()])
    kc2 = torch.stack([inp["k_cache"], inp["k_cache"]])
    vc2 = torch.stack([inp["v_cache"], inp["v_cache"]])
    K, V = torch.stack([ks1, ks2]), torch.stack([vs1, vs2])
    out = torch.full((2,) + tuple(inp["q"].shape), float("nan"), dtype=torch.float32, device="cuda")
    pa.decode_layers(out, q2, kc2, vc2, inp["block_tables"], inp["context_lens"], cfg.block_size, cfg.softmax_scale,
                     cfg.num_kv_heads, k_scale=K, v_scale=V)
    torch.cuda.synchronize()
    ref = oracle.paged_decode_layers(q2.cpu(), kc2.cpu(), vc2.cpu(), inp["block_tables"].cpu(),
                                     inp["context_lens"].cpu(), cfg.softmax_scale, cfg.num_kv_heads, K.cpu(), V.cpu(),
                                     nthreads=NTHREADS)
    err = max_abs_err(out, ref)
    log(f"[layers block scales] err32={err:.3e}")
    assert err <= TOL_F32["fp8"]


def test_validate_names_a_bad_block_scale():
    cfg = SMALL["gqa8_f16q"]
    layout, inp = setup(cfg)
    gpu_cache_write(cfg, inp)
    out = torch.full(inp["q"].shape, float("nan"), dtype=torch.float32, device="cuda")
    args = (out, inp["q"], inp["k_cache"], inp["v_cache"], inp["block_tables"], inp["context_lens"], cfg.block_size,
            cfg.softmax_scale, cfg.num_kv_heads)
    pa.decode(*args, k_scale=inp["k_scale"], v_scale=inp["v_scale"], validate=True)
    bad = inp["k_scale"].clone()
    bad[17, 3] = 0.0
    with pytest.raises(pa.PaError) as e:
        pa.decode(*args, k_scale=bad, v_scale=inp["v_scale"], validate=True)
    assert e.value.status == -9 and f"k_block_scales[{17 * cfg.num_kv_heads + 3}]" in str(e.value), str(e.value)
    bad = inp["v_scale"].clone()
    bad[0, 0] = float("nan")
    with pytest.raises(pa.PaError) as e:
        pa.cache_write(inp["k_new"], inp["v_new"], inp["k_cache"], inp["v_cache"], inp["slot_mapping"],
                       k_scale=inp["k_scale"], v_scale=bad, validate=True)
    assert e.value.status == -9 and "v_block_scales[0]" in str(e.value), str(e.value)

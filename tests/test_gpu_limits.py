"""Decode at the limits, against the fp64 oracle on every sequence:
65535 sequences (the most one launch takes) of 1-32 tokens on the
matrix-core kernel and 3000 sequences on the vector kernel, both far past
the 256 context lengths a worker reads in its first window, so the start-up
walks many windows; and 128k-token contexts on both kernels, cut across
every worker.  The work splits cover few workers (long ranges), the default,
and one unit per worker."""

import numpy as np
import pytest
import torch

import paged_kv_cache_447_amd as pa
from pa_workloads import get_config, scaled
from tests.gpu_common import (TOL_F32, TOL_OUT, gpu_cache_write, gpu_decode, host_inputs, log, max_abs_err,
                              oracle_step, setup)
from tests.test_gpu_parity import assert_counters_zero

pytestmark = pytest.mark.gpu

LIMITS = {
    "max_seqs_65535_gqa4_d64": scaled(get_config("gqa70b"), num_seqs=65535, num_heads=4, num_kv_heads=1,
                                      head_dim=64, block_size=16, num_blocks=140000, max_blocks_per_seq=2,
                                      ctx_kind="uniform", ctx_lo=1, ctx_hi=32),
    "many_seqs_3000_mha": scaled(get_config("llama7b"), num_seqs=3000, num_heads=4, num_kv_heads=4,
                                 num_blocks=12000, max_blocks_per_seq=8, ctx_kind="uniform", ctx_lo=1,
                                 ctx_hi=100),
    # 128k-token contexts: cut across every worker, so one item's merge
    # combines thousands of partials (vector kernel, fp16) ...
    "ctx_128k_mha": scaled(get_config("llama7b"), num_seqs=3, num_heads=2, num_kv_heads=2, num_blocks=11000,
                           max_blocks_per_seq=8192, ctx_kind="fixed", ctx_fixed=(131072, 5, 40000)),
    # ... and matrix-core kernel, fp8 with one scale per kv head, G = 8
    "ctx_128k_gqa8_fp8_heads": scaled(get_config("gqa70b_fp8"), num_seqs=2, num_heads=16, num_kv_heads=2,
                                      num_blocks=4200, max_blocks_per_seq=4096, ctx_kind="fixed",
                                      ctx_fixed=(131072, 777)),
}
SPLITS = [(0, 7), (0, 0), (0, 65536)]


@pytest.mark.parametrize("case", sorted(LIMITS))
def test_batch_limits_match_oracle(case):
    cfg = LIMITS[case]
    log(f"[{case}] generating")
    layout, inp = setup(cfg)
    host = host_inputs(inp)
    gpu_cache_write(cfg, inp)
    outs = []
    for part, workers in SPLITS:
        ws = pa.new_workspace(inp["q"], cfg.num_kv_heads, workers)
        out = gpu_decode(cfg, inp, partition_size=part, num_workers=workers, workspace=ws)
        out32 = gpu_decode(cfg, inp, out_dtype=torch.float32, partition_size=part, num_workers=workers,
                           workspace=ws)
        torch.cuda.synchronize()
        assert_counters_zero(ws, cfg.num_seqs, cfg.num_kv_heads)
        outs.append((workers, out, out32))
    log(f"[{case}] oracle")
    ref, _, _ = oracle_step(cfg, host)
    for workers, out, out32 in outs:
        err, err32 = max_abs_err(out, ref), max_abs_err(out32, ref)
        log(f"    workers={workers}: err={err:.3e} err32={err32:.3e} max|ref|={np.abs(ref).max():.3f}")
        assert err <= TOL_OUT[cfg.kv_dtype]
        assert err32 <= TOL_F32[cfg.kv_dtype]


def test_layers_at_the_pair_limit_match_oracle():
    """pa_decode_layers over 8 layers x 8191 sequences: 65528 (layer,
    sequence) pairs, just under the 65535 one launch takes, every output
    against the multi-layer oracle."""
    from pa_workloads import make_layout
    from pa_workloads.layers import LayerConfig, make_layer_inputs
    from tests.test_gpu_layers import gpu_layer_step, oracle_layer_step

    lcfg = LayerConfig("max_pairs_8x8191",
                       scaled(get_config("gqa70b"), num_seqs=8191, num_heads=4, num_kv_heads=1, head_dim=64,
                              block_size=16, num_blocks=16500, max_blocks_per_seq=2, ctx_kind="uniform", ctx_lo=1,
                              ctx_hi=32), 8)
    cfg = lcfg.base
    log(f"[{lcfg.name}] generating")
    inp = make_layer_inputs(lcfg, make_layout(cfg), "cuda")
    host = host_inputs(inp)
    ws = pa.new_workspace(inp["q"], cfg.num_kv_heads)
    out = gpu_layer_step(lcfg, inp, out_dtype=torch.float32, workspace=ws)
    torch.cuda.synchronize()
    assert_counters_zero(ws, lcfg.num_layers * cfg.num_seqs, cfg.num_kv_heads)
    log(f"[{lcfg.name}] oracle")
    ref, _, _ = oracle_layer_step(lcfg, host)
    err32 = max_abs_err(out, ref)
    log(f"    err32={err32:.3e} max|ref|={np.abs(ref).max():.3f}")
    assert err32 <= TOL_F32[cfg.kv_dtype]

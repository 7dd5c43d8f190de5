"""Device contents are trusted but cannot make a kernel reach outside its
buffers: block-table entries outside [0, num_blocks) and context lengths
outside [0, max_blocks_per_seq * block_size] are clamped, so only the
sequence that holds them gets an unspecified result.

One sequence gets garbage table entries (negative, past the pool, the int32
extremes), one a context length of INT32_MAX and one of -5.  Every other
sequence must come out exactly as in a clean run: bit for bit when the decode
unit is the table's whole width (each sequence is one unit, so nothing is cut
and no other sequence's length moves a cut), and within the usual bound of the
oracle with the default split.  Prefill computes each
(sequence, kv head) pair whole in one workgroup, so its other rows must match
the clean run bit for bit."""

import numpy as np
import pytest
import torch

import paged_kv_cache_447_amd as pa
from tests.gpu_common import TOL_F32, gpu_cache_write, gpu_decode, host_inputs, log, max_abs_err, oracle_step, setup
from tests.test_gpu_parity import SMALL as DECODE_CASES
from tests.test_gpu_prefill import CASES as PREFILL_CASES, setup as prefill_setup

pytestmark = pytest.mark.gpu

I32_MIN, I32_MAX = -(2**31), 2**31 - 1


def _poison(block_tables, context_lens, num_blocks):
    """Garbage in sequences 1, 2 and 3; returns the indices of the others."""
    bt, cl = block_tables.clone(), context_lens.clone()
    W = bt.shape[1]
    junk = torch.tensor([-7, num_blocks, num_blocks + 1000, I32_MAX, I32_MIN, -1], dtype=torch.int32)
    bt[1] = junk.repeat((W + len(junk) - 1) // len(junk))[:W].to(bt.device)
    cl[2] = I32_MAX
    cl[3] = -5
    good = [i for i in range(bt.shape[0]) if i not in (1, 2, 3)]
    return bt, cl, good


@pytest.mark.parametrize("case", ["mha_f16_edges", "gqa8_f16", "fp8_gqa4_d64"])
def test_decode_garbage_stays_in_its_sequence(case):
    cfg = DECODE_CASES[case]
    log(f"[untrusted decode {case}]")
    _, inp = setup(cfg)
    host = host_inputs(inp)
    gpu_cache_write(cfg, inp)
    bt, cl, good = _poison(inp["block_tables"], inp["context_lens"], cfg.num_blocks)
    dirty_inp = dict(inp, block_tables=bt, context_lens=cl)

    whole = cfg.max_blocks_per_seq * cfg.block_size
    clean1 = gpu_decode(cfg, inp, out_dtype=torch.float32, partition_size=whole)
    dirty1 = gpu_decode(cfg, dirty_inp, out_dtype=torch.float32, partition_size=whole)
    dirty = gpu_decode(cfg, dirty_inp, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(dirty1[good].view(torch.int32), clean1[good].view(torch.int32))

    ref, _, _ = oracle_step(cfg, host)
    err = max_abs_err(dirty[good], ref[good])
    log(f"    other sequences: bit-identical with whole-sequence units; default split err32={err:.3e}")
    assert err <= TOL_F32[cfg.kv_dtype]


@pytest.mark.parametrize("case", ["whole_prompt_gqa2", "verify_gqa8"])
def test_prefill_garbage_stays_in_its_sequence(case):
    pcfg = PREFILL_CASES[case]
    cfg = pcfg.base
    log(f"[untrusted prefill {case}]")
    assert cfg.num_seqs >= 5
    _, inp = prefill_setup(pcfg)
    pa.cache_write(inp["k_new"], inp["v_new"], inp["k_cache"], inp["v_cache"], inp["slot_mapping"],
                   k_scale=inp["k_scale"], v_scale=inp["v_scale"])
    bt, cl, good = _poison(inp["block_tables"], inp["context_lens"], cfg.num_blocks)

    def run(block_tables, context_lens):
        out = torch.empty(inp["q"].shape, dtype=torch.float32, device=inp["q"].device)
        pa.prefill(out, inp["q"], inp["k_cache"], inp["v_cache"], block_tables, context_lens,
                   inp["query_start_loc"], cfg.block_size, cfg.softmax_scale, cfg.num_kv_heads,
                   k_scale=inp["k_scale"], v_scale=inp["v_scale"])
        return out

    clean = run(inp["block_tables"], inp["context_lens"])
    dirty = run(bt, cl)
    torch.cuda.synchronize()
    qsl = inp["query_start_loc"].cpu().numpy()
    rows = np.concatenate([np.arange(qsl[i], qsl[i + 1]) for i in good])
    rows_t = torch.from_numpy(rows).to(clean.device)
    assert torch.equal(dirty[rows_t].view(torch.int32), clean[rows_t].view(torch.int32))
    log(f"    {len(rows)} rows of the other sequences bit-identical to the clean run")

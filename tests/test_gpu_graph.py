"""A serving step captured in a HIP graph (torch.cuda.graph) and replayed.

The cache write followed by decode (one layer or several), or by prefill, goes through the C ABI into
caller-owned workspaces and outputs, so the graph holds kernel launches only:
no allocation and no memset.  The kernels leave their merge and hand-out
counters at zero, so the same workspace serves every replay.  Each replay,
with eager calls, in-place input changes and synchronisations between
replays, must give the same bits as the eager calls on the same inputs."""

import pytest
import torch

import paged_kv_cache_447_amd as pa
from tests.gpu_common import gpu_cache_write, gpu_decode, log, setup
from tests.test_gpu_head_scales import SMALL as HEAD_SCALE_CASES
from tests.test_gpu_parity import SMALL as DECODE_CASES, assert_counters_zero
from tests.test_gpu_prefill import CASES as PREFILL_CASES, setup as prefill_setup

pytestmark = pytest.mark.gpu

REPLAYS = 4

DECODE = {
    "mha_f16_edges": DECODE_CASES["mha_f16_edges"],          # vector-ALU kernel, G = 1
    "gqa8_f16": DECODE_CASES["gqa8_f16"],                    # matrix-core kernel, LDS ring
    "fp8_heads_gqa4_d64": HEAD_SCALE_CASES["gqa4_f16q_d64_bs16"],  # fp8, one scale per kv head
}


def _other_q(q):
    """A second query of the same shape (the first one reversed along the
    sequences and negated), so replays can be told apart."""
    return (-q.flip(0)).contiguous()


@pytest.mark.parametrize("case", sorted(DECODE))
def test_decode_step_replays_in_a_graph(case):
    cfg = DECODE[case]
    log(f"[graph decode {case}]")
    _, inp = setup(cfg)
    ws = pa.new_workspace(inp["q"], cfg.num_kv_heads)
    q_a = inp["q"].clone()
    q_b = _other_q(q_a)

    # eager results on both queries (the write is idempotent: same slots, same values)
    gpu_cache_write(cfg, inp)
    ref_a = gpu_decode(cfg, inp, workspace=ws).clone()
    inp["q"].copy_(q_b)
    ref_b = gpu_decode(cfg, inp, workspace=ws).clone()
    torch.cuda.synchronize()
    assert not torch.equal(ref_a, ref_b)

    out = torch.empty_like(ref_a)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gpu_cache_write(cfg, inp)
        gpu_decode(cfg, inp, out=out, workspace=ws)
    torch.cuda.synchronize()
    assert_counters_zero(ws, cfg.num_seqs, cfg.num_kv_heads)

    for r in range(REPLAYS):
        use_a = r % 2 == 0
        inp["q"].copy_(q_a if use_a else q_b)
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_a if use_a else ref_b), f"replay {r} differs from the eager call"
        assert_counters_zero(ws, cfg.num_seqs, cfg.num_kv_heads)
        # eager work on the same workspace between replays
        eager = gpu_decode(cfg, inp, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(eager, ref_a if use_a else ref_b)
    log(f"    {REPLAYS} replays bit-identical to the eager calls")


@pytest.mark.parametrize("case", ["small_gqa4_d64", "verify_gqa8", "fp8_heads_verify_gqa8"])
def test_prefill_step_replays_in_a_graph(case):
    """Column mode (prompt chunks) and key-split mode (verification, pairs
    handed out through the workspace counter)."""
    pcfg = PREFILL_CASES[case]
    cfg = pcfg.base
    log(f"[graph prefill {case}]")
    _, inp = prefill_setup(pcfg)
    ws = pa.new_prefill_workspace(inp["q"].device)
    q_a = inp["q"].clone()
    q_b = _other_q(q_a)

    def write():
        pa.cache_write(inp["k_new"], inp["v_new"], inp["k_cache"], inp["v_cache"], inp["slot_mapping"],
                       k_scale=inp["k_scale"], v_scale=inp["v_scale"])

    def prefill(out):
        pa.prefill(out, inp["q"], inp["k_cache"], inp["v_cache"], inp["block_tables"], inp["context_lens"],
                   inp["query_start_loc"], cfg.block_size, cfg.softmax_scale, cfg.num_kv_heads,
                   k_scale=inp["k_scale"], v_scale=inp["v_scale"], workspace=ws)
        return out

    write()
    ref_a = prefill(torch.empty_like(q_a))
    inp["q"].copy_(q_b)
    ref_b = prefill(torch.empty_like(q_a))
    torch.cuda.synchronize()
    assert not torch.equal(ref_a, ref_b)

    out = torch.empty_like(q_a)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        write()
        prefill(out)
    torch.cuda.synchronize()

    for r in range(REPLAYS):
        use_a = r % 2 == 0
        inp["q"].copy_(q_a if use_a else q_b)
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_a if use_a else ref_b), f"replay {r} differs from the eager call"
        assert int(ws.view(torch.int32)[0]) == 0, "the pair counter is left at zero"
        eager = prefill(torch.empty_like(q_a))
        torch.cuda.synchronize()
        assert torch.equal(eager, ref_a if use_a else ref_b)
    log(f"    {REPLAYS} replays bit-identical to the eager calls")


@pytest.mark.parametrize("case", ["gqa8_bf16", "fp8_gqa4_d64"])
def test_layers_step_replays_in_a_graph(case):
    """pa_decode_layers after the cache write of every layer's new token,
    captured once and replayed like the single-layer step."""
    from pa_workloads import make_layout
    from pa_workloads.layers import flat_slots, make_layer_inputs
    from tests.test_gpu_layers import SMALL as LAYER_CASES

    lcfg = LAYER_CASES[case]
    cfg = lcfg.base
    L, NB, bs = lcfg.num_layers, cfg.num_blocks, cfg.block_size
    log(f"[graph layers {case}]")
    inp = make_layer_inputs(lcfg, make_layout(cfg), "cuda")
    ws = pa.new_workspace(inp["q"], cfg.num_kv_heads)
    kc = inp["k_cache"].view((L * NB,) + tuple(inp["k_cache"].shape[2:]))
    vc = inp["v_cache"].view((L * NB,) + tuple(inp["v_cache"].shape[2:]))
    kn = inp["k_new"].reshape((-1,) + tuple(inp["k_new"].shape[2:]))
    vn = inp["v_new"].reshape((-1,) + tuple(inp["v_new"].shape[2:]))
    slots = flat_slots(inp["slot_mapping"], L, NB * bs)
    q_a = inp["q"].clone()
    q_b = (-q_a.flip(1)).contiguous()

    def step(out):
        pa.cache_write(kn, vn, kc, vc, slots, k_scale=inp["k_scale"], v_scale=inp["v_scale"])
        pa.decode_layers(out, inp["q"], inp["k_cache"], inp["v_cache"], inp["block_tables"], inp["context_lens"],
                         bs, cfg.softmax_scale, cfg.num_kv_heads, k_scale=inp["k_scale"], v_scale=inp["v_scale"],
                         workspace=ws)
        return out

    ref_a = step(torch.empty_like(q_a))
    inp["q"].copy_(q_b)
    ref_b = step(torch.empty_like(q_a))
    torch.cuda.synchronize()
    assert not torch.equal(ref_a, ref_b)

    out = torch.empty_like(q_a)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(out)
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        use_a = r % 2 == 0
        inp["q"].copy_(q_a if use_a else q_b)
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_a if use_a else ref_b), f"replay {r} differs from the eager call"
        assert_counters_zero(ws, L * cfg.num_seqs, cfg.num_kv_heads)
        eager = step(torch.empty_like(q_a))
        torch.cuda.synchronize()
        assert torch.equal(eager, ref_a if use_a else ref_b)
    log(f"    {REPLAYS} replays bit-identical to the eager calls")


def test_copy_on_write_then_decode_replays_in_a_graph():
    """pa_copy_blocks (a private copy of sequence 0's last block, inside the
    pool) then decode through a table that points at the copy, captured once.
    Before every replay the copy's block is poisoned with NaN, so each replay
    must redo the copy; its output must equal the eager decode of the
    original table bit for bit."""
    cfg = DECODE_CASES["gqa8_f16"]
    log("[graph copy-on-write + decode gqa8_f16]")
    _, inp = setup(cfg)
    gpu_cache_write(cfg, inp)
    bt = inp["block_tables"]
    ctx0 = int(inp["context_lens"][0])
    j = (ctx0 - 1) // cfg.block_size
    used = set(bt.flatten().tolist())
    new = next(b for b in range(cfg.num_blocks - 1, -1, -1) if b not in used)
    old = int(bt[0, j])
    bt_copy = bt.clone()
    bt_copy[0, j] = new
    mapping = torch.tensor([[old, new]], dtype=torch.int64, device=bt.device)
    ws = pa.new_workspace(inp["q"], cfg.num_kv_heads)
    q_a = inp["q"].clone()
    q_b = _other_q(q_a)

    ref_a = gpu_decode(cfg, inp, workspace=ws).clone()
    inp["q"].copy_(q_b)
    ref_b = gpu_decode(cfg, inp, workspace=ws).clone()
    torch.cuda.synchronize()

    copied = dict(inp, block_tables=bt_copy)
    out = torch.empty_like(ref_a)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pa.copy_blocks(inp["k_cache"], inp["v_cache"], inp["k_cache"], inp["v_cache"], mapping)
        gpu_decode(cfg, copied, out=out, workspace=ws)
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        use_a = r % 2 == 0
        inp["q"].copy_(q_a if use_a else q_b)
        inp["k_cache"][new].fill_(float("nan"))
        inp["v_cache"][new].fill_(float("nan"))
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_a if use_a else ref_b), f"replay {r} differs from the eager call"
        # byte comparison: the pool's unwritten slots hold NaN on purpose
        assert torch.equal(inp["k_cache"][new].view(torch.int16), inp["k_cache"][old].view(torch.int16))
        assert torch.equal(inp["v_cache"][new].view(torch.int16), inp["v_cache"][old].view(torch.int16))
        assert_counters_zero(ws, cfg.num_seqs, cfg.num_kv_heads)
    log(f"    {REPLAYS} replays bit-identical to the eager calls")


def test_swap_out_replays_in_a_graph():
    """pa_copy_blocks from the device pool into pinned host pools, captured
    once.  The host pools are cleared on the CPU before every replay; each
    replay must write the mapped blocks back, byte for byte."""
    cfg = DECODE_CASES["gqa8_f16"]
    log("[graph swap-out gqa8_f16]")
    _, inp = setup(cfg)
    gpu_cache_write(cfg, inp)
    torch.cuda.synchronize()
    n_host = 40
    src = torch.randperm(cfg.num_blocks, generator=torch.Generator().manual_seed(7))[:n_host]
    mapping = torch.stack([src, torch.arange(n_host)], dim=1).to(torch.int64).cuda()
    shape = (n_host,) + tuple(inp["k_cache"].shape[1:])
    hk = torch.empty(shape, dtype=inp["k_cache"].dtype).pin_memory()
    hv = torch.empty(shape, dtype=inp["v_cache"].dtype).pin_memory()
    want_k = inp["k_cache"][src.cuda()].cpu().view(torch.int16)
    want_v = inp["v_cache"][src.cuda()].cpu().view(torch.int16)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pa.copy_blocks(hk, hv, inp["k_cache"], inp["v_cache"], mapping)
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        hk.zero_()
        hv.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(hk.view(torch.int16), want_k), f"replay {r}: K blocks differ"
        assert torch.equal(hv.view(torch.int16), want_v), f"replay {r}: V blocks differ"
    log(f"    {REPLAYS} replays wrote the {n_host} blocks back")

"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Every expected value comes from the oracle or from the generator's own bytes,
never from the HIP path.  Run on an MI355X with ``pytest -m gpu``.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_447_amd as pa
from pa_workloads import get_config, make_inputs, make_layout, scaled
from pa_workloads.configs import CONFIG_ORDER
from tests.gpu_common import (TOL_F32, TOL_OUT, gpu_cache_write, gpu_decode, host_inputs, log, max_abs_err,
                              oracle_step, setup)

pytestmark = pytest.mark.gpu


def _bytes(t):
    return t.detach().cpu().contiguous().view(torch.uint8)


@pytest.mark.parametrize("name", CONFIG_ORDER)
def test_full_size_step_matches_oracle(name):
    """One decode step of each workload at full size: cache write (bit-exact over the
    whole pool) then decode (q-dtype and fp32 outputs) against the oracle."""
    cfg = get_config(name)
    log(f"[{name}] generating")
    layout, inp = setup(cfg)
    host = host_inputs(inp)
    log(f"[{name}] gpu step")
    gpu_cache_write(cfg, inp)
    out = gpu_decode(cfg, inp)
    out32 = gpu_decode(cfg, inp, out_dtype=torch.float32)
    torch.cuda.synchronize()
    log(f"[{name}] oracle")
    ref, kc, vc = oracle_step(cfg, host)
    assert torch.equal(_bytes(inp["k_cache"]), kc.view(torch.uint8)), "k_cache differs from the oracle's write"
    assert torch.equal(_bytes(inp["v_cache"]), vc.view(torch.uint8)), "v_cache differs from the oracle's write"
    err = max_abs_err(out, ref)
    err32 = max_abs_err(out32, ref)
    log(f"[{name}] max|err| out={err:.3e} (tol {TOL_OUT[cfg.kv_dtype]})  fp32-out={err32:.3e} "
        f"(tol {TOL_F32[cfg.kv_dtype]})  max|ref|={np.abs(ref).max():.3f}")
    assert err <= TOL_OUT[cfg.kv_dtype]
    assert err32 <= TOL_F32[cfg.kv_dtype]


SMALL = {
    # ragged lengths around block and partition edges, a full table row, GQA groups
    "mha_f16_edges": scaled(get_config("llama7b"), num_seqs=12, num_blocks=600, max_blocks_per_seq=40,
                            ctx_kind="fixed", ctx_fixed=(1, 2, 15, 16, 17, 255, 256, 257, 511, 512, 513, 640)),
    "mha_bf16_d64": scaled(get_config("llama13b_prefix"), num_seqs=16, num_heads=6, num_kv_heads=6, head_dim=64,
                           num_blocks=900, max_blocks_per_seq=64, ctx_lo=512, ctx_hi=1024, share_group=4),
    "gqa2_f16": scaled(get_config("gqa70b"), num_seqs=9, num_heads=8, num_kv_heads=4, num_blocks=2000,
                       max_blocks_per_seq=48, ctx_hi=1536),
    "gqa4_bf16_bs16": scaled(get_config("gqa70b"), num_seqs=7, num_heads=16, num_kv_heads=4, block_size=16,
                             kv_dtype="bf16", q_dtype="bf16", num_blocks=3000, max_blocks_per_seq=96, ctx_hi=1536),
    "gqa8_f16": scaled(get_config("gqa70b"), num_seqs=10, num_blocks=2000, max_blocks_per_seq=64, ctx_hi=2048),
    "fp8_bf16q": scaled(get_config("fp8_long"), num_seqs=4, num_heads=8, num_kv_heads=8, q_dtype="bf16",
                        num_blocks=1200, max_blocks_per_seq=256, ctx_lo=1, ctx_hi=4096, partition_size=256),
    "fp8_gqa4_d64": scaled(get_config("fp8_long"), num_seqs=5, num_heads=16, num_kv_heads=4, head_dim=64,
                           num_blocks=800, max_blocks_per_seq=128, ctx_lo=100, ctx_hi=2048, partition_size=0),
    "f32_d128_bs32": scaled(get_config("tiny"), num_seqs=6, num_heads=4, num_kv_heads=2, head_dim=128,
                            block_size=32, num_blocks=100, max_blocks_per_seq=10, ctx_kind="uniform", ctx_lo=1,
                            ctx_hi=320, scale=None),
    "full_row": scaled(get_config("llama7b"), num_seqs=3, num_blocks=200, max_blocks_per_seq=20,
                       ctx_kind="fixed", ctx_fixed=(320, 319, 1)),
    "gqa16_f16": scaled(get_config("gqa70b"), num_seqs=6, num_heads=32, num_kv_heads=2, num_blocks=600,
                        max_blocks_per_seq=48, ctx_hi=1536),
    "gqa8_bf16_d64": scaled(get_config("gqa70b"), num_seqs=8, num_heads=32, num_kv_heads=4, head_dim=64,
                            kv_dtype="bf16", q_dtype="bf16", num_blocks=800, max_blocks_per_seq=40, ctx_hi=1280),
    "gqa16_fp8_bf16q": scaled(get_config("fp8_long"), num_seqs=5, num_heads=32, num_kv_heads=2, q_dtype="bf16",
                              num_blocks=1000, max_blocks_per_seq=160, ctx_lo=1, ctx_hi=2560, partition_size=0),
}


# (partition_size, num_workers): the unit of work and how many wavefronts share
# it decide where contexts are cut and merged.  One worker cuts nothing; a
# handful of workers cut long contexts into a few big segments; many workers
# (more than there are units, for the small cases) give one unit each.
SPLITS = [(0, 0), (64, 0), (256, 0), (0, 4), (0, 36), (16, 100), (0, 65536)]


@pytest.mark.parametrize("case", sorted(SMALL))
@pytest.mark.parametrize("split", SPLITS, ids=[f"p{p}w{w}" for p, w in SPLITS])
def test_small_cases_match_oracle(case, split):
    cfg = SMALL[case]
    partition, workers = split
    part = partition if partition % cfg.block_size == 0 else 0
    log(f"[{case} p={part} w={workers}]")
    layout, inp = setup(cfg)
    host = host_inputs(inp)
    gpu_cache_write(cfg, inp)
    ws = pa.new_workspace(inp["q"], cfg.num_kv_heads, workers)
    out = gpu_decode(cfg, inp, partition_size=part, num_workers=workers, workspace=ws)
    out32 = gpu_decode(cfg, inp, out_dtype=torch.float32, partition_size=part, num_workers=workers, workspace=ws)
    torch.cuda.synchronize()
    ref, kc, vc = oracle_step(cfg, host)
    assert torch.equal(_bytes(inp["k_cache"]), kc.view(torch.uint8))
    assert torch.equal(_bytes(inp["v_cache"]), vc.view(torch.uint8))
    err, err32 = max_abs_err(out, ref), max_abs_err(out32, ref)
    log(f"    err={err:.3e} err32={err32:.3e}")
    assert err <= TOL_OUT[cfg.kv_dtype]
    assert err32 <= TOL_F32[cfg.kv_dtype]
    # every call leaves the merge counters at zero for the next one
    assert_counters_zero(ws, cfg.num_seqs, cfg.num_kv_heads)


def counters_view(ws, S, Hkv):
    """The merge counters of a decode over S (layer, sequence) pairs: the last
    round_up(4 S Hkv, 256) bytes of the workspace rounded down to 256."""
    end = ws.numel() // 256 * 256
    n = (4 * S * Hkv + 255) // 256 * 256
    return ws[end - n:end - n + 4 * S * Hkv].view(torch.int32)


def assert_counters_zero(ws, S, Hkv):
    assert int(counters_view(ws, S, Hkv).abs().sum()) == 0


@pytest.mark.parametrize("name,G,kv_dtype,workers", [("gqa70b", 8, "f16", 64), ("gqa70b", 4, "bf16", 100),
                                                     ("gqa70b", 16, "f16", 32), ("gqa70b", 8, "f16", 0)])
def test_few_workers_match_oracle_and_repeat_exactly(name, G, kv_dtype, workers):
    """Grouped-query shapes on the matrix-core path with few workers for the
    work (long ranges, many segments each, the load ring running across
    segment boundaries): the results match the oracle, repeat bit for bit, and
    the merge counters are back at zero after every call."""
    cfg = scaled(get_config(name), num_seqs=24)
    cfg = scaled(cfg, num_heads=cfg.num_kv_heads * G, kv_dtype=kv_dtype, q_dtype=kv_dtype)
    log(f"[{name} G={G} {kv_dtype} workers={workers}]")
    layout, inp = setup(cfg)
    host = host_inputs(inp)
    gpu_cache_write(cfg, inp)
    ref, _, _ = oracle_step(cfg, host)
    ws = pa.new_workspace(inp["q"], cfg.num_kv_heads, workers)
    outs = []
    for _ in range(3):
        outs.append(gpu_decode(cfg, inp, out_dtype=torch.float32, num_workers=workers, workspace=ws))
        torch.cuda.synchronize()
        assert_counters_zero(ws, cfg.num_seqs, cfg.num_kv_heads)
    e = max_abs_err(outs[0], ref)
    log(f"    err32={e:.3e}")
    assert e <= TOL_F32[cfg.kv_dtype]
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int32), outs[0].view(torch.int32))


@pytest.mark.parametrize("name", ["llama7b", "gqa70b", "fp8_long"])
def test_split_choices_agree(name):
    """Split-context is a re-association of the same softmax: every work unit and
    worker count gives the oracle's answer (fp32 output), and they agree with
    each other."""
    cfg = get_config(name)
    if name != "fp8_long":
        cfg = scaled(cfg, num_seqs=16)
    layout, inp = setup(cfg)
    host = host_inputs(inp)
    gpu_cache_write(cfg, inp)
    ref, _, _ = oracle_step(cfg, host)
    outs = {}
    for p, w in ((0, 0), (cfg.block_size, 0), (256, 0), (1024, 0), (0, 1), (0, 52), (512, 1000),
                 (cfg.max_blocks_per_seq * cfg.block_size, 0)):
        outs[(p, w)] = gpu_decode(cfg, inp, out_dtype=torch.float32, partition_size=p, num_workers=w)
    torch.cuda.synchronize()
    for (p, w), o in outs.items():
        e = max_abs_err(o, ref)
        log(f"[{name}] partition {p} workers {w}: err32={e:.3e}")
        assert e <= TOL_F32[cfg.kv_dtype]
    first = next(iter(outs.values())).double()
    for o in outs.values():
        assert float((o.double() - first).abs().max()) <= TOL_F32[cfg.kv_dtype]


@pytest.mark.parametrize("kv_dtype,G,bs", [("f32", 1, 16), ("f16", 1, 16), ("bf16", 1, 32), ("f16", 8, 32),
                                           ("bf16", 4, 16), ("fp8", 1, 16), ("f16", 2, 16), ("fp8", 16, 32),
                                           ("f32", 8, 16)])
def test_needle_block_resolution_is_bit_exact(kv_dtype, G, bs):
    """Plant one key per sequence that dominates every other score by > 200 nats: the
    output must then be that token's V row, bit for bit -- for every needle position,
    with and without split partitions."""
    Hkv = 2
    base = get_config("fp8_long" if kv_dtype == "fp8" else "llama7b")
    cfg = scaled(base, num_seqs=6, num_heads=Hkv * G, num_kv_heads=Hkv, block_size=bs,
                 kv_dtype=kv_dtype, q_dtype="f16" if kv_dtype == "fp8" else kv_dtype,
                 num_blocks=1200, max_blocks_per_seq=2048 // bs, ctx_kind="fixed",
                 ctx_fixed=(1, bs, bs + 1, 300, 1025, 2048), partition_size=0)
    layout, inp = setup(cfg)
    host = host_inputs(inp)
    # every stored token, the new ones included, as the oracle's cache write leaves the pool
    kc_h, vc_h = oracle.cache_write(host["k_new"], host["v_new"], host["k_cache"], host["v_cache"],
                                    host["slot_mapping"], host["k_scale"], host["v_scale"], inplace=True)
    inp["k_cache"], inp["v_cache"] = kc_h.cuda(), vc_h.cuda()
    q = inp["q"]
    for s in range(cfg.num_seqs):  # one query direction per group, so one key can dominate for all G heads
        for kvh in range(Hkv):
            q[s, kvh * G:(kvh + 1) * G] = q[s, kvh * G]
    bt = layout.block_tables
    ctx = layout.context_lens
    k_scale = 1.0 if kv_dtype == "fp8" else inp["k_scale"]
    rng = np.random.default_rng(3)
    for rnd in range(5):
        kc = inp["k_cache"].clone()
        expected = torch.empty(q.shape, dtype=torch.float32)
        for s in range(cfg.num_seqs):
            L = int(ctx[s])
            choices = [0, L - 1, min(L - 1, bs - 1), min(L - 1, bs), min(L - 1, 255), min(L - 1, 256),
                       int(rng.integers(L))]
            t = choices[rnd % len(choices)] if rnd < 4 else choices[-1]
            phys, off = int(bt[s, t // bs]), t % bs
            for kvh in range(Hkv):
                qv = q[s, kvh * G].float()
                if kv_dtype == "fp8":
                    codes = torch.where(qv >= 0, 0x7E, 0xFE).to(torch.uint8)
                    kc.view(torch.uint8)[phys, off, kvh] = codes
                    vrow = vc_h[phys, off, kvh].float() * torch.tensor(inp["v_scale"], dtype=torch.float32)
                else:
                    c = 300.0 / (cfg.softmax_scale * float(qv.norm()))
                    kc[phys, off, kvh] = (c * qv / qv.norm()).to(kc.dtype)
                    vrow = vc_h[phys, off, kvh].float()
                expected[s, kvh * G:(kvh + 1) * G] = vrow
        for part, workers in ((0, 0), (bs, 0), (256, 0), (0, 1), (bs, 24)):
            out = torch.empty_like(q)
            pa.decode(out, q, kc, inp["v_cache"], inp["block_tables"], inp["context_lens"], bs, cfg.softmax_scale,
                      Hkv, k_scale=k_scale, v_scale=inp["v_scale"], partition_size=part, num_workers=workers)
            torch.cuda.synchronize()
            want = expected.to(q.dtype)
            got = out.cpu()
            assert torch.equal(got.view(torch.int16) if got.dtype != torch.float32 else got.view(torch.int32),
                               want.view(torch.int16) if want.dtype != torch.float32 else want.view(torch.int32)), \
                f"round {rnd} partition {part} workers {workers}"


@pytest.mark.parametrize("q_dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("G", [1, 4])
def test_fp8_hardware_decode_matches_ocp_table(q_dtype, G):
    """ctx = 1 makes out = V exactly: put all 256 codes in V rows and read them back in fp32,
    through the vector path (G = 1) and the matrix-core path (G = 4), for both query types."""
    D, bs = 128, 16
    dev = "cuda"
    kc = torch.zeros((4, bs, 1, D), dtype=torch.uint8, device=dev)
    vc = torch.zeros((4, bs, 1, D), dtype=torch.uint8, device=dev)
    vc[0, 0, 0] = torch.arange(0, 128, dtype=torch.int32).to(torch.uint8).to(dev)
    vc[1, 0, 0] = torch.arange(128, 256, dtype=torch.int32).to(torch.uint8).to(dev)
    bt = torch.tensor([[0], [1]], dtype=torch.int32, device=dev)
    cl = torch.tensor([1, 1], dtype=torch.int32, device=dev)
    q = torch.randn((2, G, D), device=dev).to(q_dtype)
    out = torch.empty((2, G, D), dtype=torch.float32, device=dev)
    pa.decode(out, q, kc.view(torch.float8_e4m3fn), vc.view(torch.float8_e4m3fn), bt, cl, bs, 0.1, 1)
    got = out.cpu()[:, 0].reshape(-1).numpy()
    for g in range(1, G):
        assert torch.equal(out[:, g].cpu().view(torch.int32), out[:, 0].cpu().view(torch.int32))
    for code in range(256):
        want = oracle.fp8_to_double(code)
        if math.isnan(want):
            assert math.isnan(got[code])
        else:
            assert got[code] == np.float32(want), (code, got[code], want)


def test_repeated_runs_are_bit_identical():
    cfg = scaled(get_config("gqa70b"), num_seqs=24)
    layout, inp = setup(cfg)
    gpu_cache_write(cfg, inp)
    a = gpu_decode(cfg, inp)
    b = gpu_decode(cfg, inp)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_tiny_round_trip_before_and_after_the_write():
    """Decode the tiny workload over ctx-1 tokens (the new slots still hold NaN and
    must not be read), write the 4 new tokens, decode over ctx."""
    cfg = get_config("tiny")
    layout, inp = setup(cfg)
    host = host_inputs(inp)
    before = torch.clamp(inp["context_lens"] - 1, min=0)
    out0 = gpu_decode(cfg, inp, context_lens=before)
    torch.cuda.synchronize()
    ref0 = oracle.paged_decode(host["q"], host["k_cache"], host["v_cache"], host["block_tables"], before.cpu(),
                               cfg.softmax_scale, cfg.num_kv_heads)
    assert max_abs_err(out0, ref0) <= TOL_F32["f32"]
    assert (out0[0] == 0).all()  # ctx 1 -> 0 before the write
    gpu_cache_write(cfg, inp)
    out1 = gpu_decode(cfg, inp)
    torch.cuda.synchronize()
    ref1, _, _ = oracle_step(cfg, host)
    assert max_abs_err(out1, ref1) <= TOL_F32["f32"]


def test_empty_batch_and_zero_length_sequences():
    cfg = scaled(get_config("llama7b"), num_seqs=4, num_blocks=300)
    layout, inp = setup(cfg)
    gpu_cache_write(cfg, inp)  # each sequence's last slot holds poison until its token is written
    out = torch.full_like(inp["q"], 7.0)
    cl = inp["context_lens"].clone()
    cl[1] = 0
    cl[3] = 0
    gpu_decode(cfg, inp, context_lens=cl, out=out)
    torch.cuda.synchronize()
    assert (out[1] == 0).all() and (out[3] == 0).all()
    assert torch.isfinite(out).all()
    empty = inp["q"][:0]
    pa.decode(torch.empty_like(empty), empty, inp["k_cache"], inp["v_cache"], inp["block_tables"][:0],
              inp["context_lens"][:0], cfg.block_size, cfg.softmax_scale, cfg.num_kv_heads)


def test_side_stream_and_strided_query():
    cfg = scaled(get_config("llama7b"), num_seqs=8, num_blocks=800)
    layout, inp = setup(cfg)
    host = host_inputs(inp)
    gpu_cache_write(cfg, inp)
    S, H, D = inp["q"].shape
    big = torch.zeros((S, 3 * H, D), dtype=inp["q"].dtype, device="cuda")
    big[:, H:2 * H] = inp["q"]
    inp["q"] = big[:, H:2 * H]  # a view: sequence stride 3*H*D
    out_big = torch.zeros((S, 2, H, D), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        gpu_decode(cfg, inp, out=out_big[:, 1])
    side.synchronize()
    ref, _, _ = oracle_step(cfg, host)
    assert max_abs_err(out_big[:, 1], ref) <= TOL_F32["f16"]
    assert (out_big[:, 0] == 0).all()


def test_cache_write_skip_rules_and_int32_slots():
    NB, bs, Hkv, D = 8, 16, 2, 128
    g = torch.Generator(device="cuda").manual_seed(5)
    kc = torch.randn((NB, bs, Hkv, D), generator=g, device="cuda").half()
    vc = torch.randn((NB, bs, Hkv, D), generator=g, device="cuda").half()
    k = torch.randn((5, Hkv, D), generator=g, device="cuda").half()
    v = torch.randn((5, Hkv, D), generator=g, device="cuda").half()
    slots = torch.tensor([3, -1, NB * bs, 127, 17], dtype=torch.int32, device="cuda")
    hk, hv = kc.cpu(), vc.cpu()
    pa.cache_write(k, v, kc, vc, slots)
    torch.cuda.synchronize()
    keep = torch.tensor([0, 3, 4])
    ek, ev = oracle.cache_write(k.cpu()[keep], v.cpu()[keep], hk, hv, slots.cpu().long()[keep])
    assert torch.equal(kc.cpu().view(torch.int16), ek.view(torch.int16))
    assert torch.equal(vc.cpu().view(torch.int16), ev.view(torch.int16))


@pytest.mark.parametrize("in_dtype", [torch.float16, torch.bfloat16, torch.float32])
def test_fp8_cache_write_rounding_edges(in_dtype):
    """Ties, subnormals, saturation and NaN through the kernel's quantiser, bit
    for bit, with a power-of-two scale (the division by it is exact) and with
    scale = fp32(1/3), where the stored values sit at and one or two steps of
    the input dtype around midpoint * scale, so the quotient lands within a few
    fp32 ulps of an e4m3fn midpoint and the division's own rounding decides the
    tie (both sides divide in fp32, as the cache write is defined)."""
    grid = [oracle.fp8_to_double(c) for c in range(0x7F)]
    # power-of-two scale: exact midpoints, just above codes, saturation, specials
    vals = []
    for c in range(0x7E):
        vals.append((grid[c] + grid[c + 1]) / 2)  # exact midpoints -> ties to even
        vals.append(grid[c] * 1.0001)
    vals += [448.0, 460.0, 470.0, 1e4, float("inf"), float("nan"), 0.0, -0.0, 2.0**-12, 2.0**-10, 3 * 2.0**-11]
    x = torch.tensor(vals, dtype=torch.float64)
    _check_quantiser(in_dtype, 0.5, (torch.cat([x, -x]) * 0.5).to(in_dtype))
    # non-power-of-two scale: stored values around every midpoint times the scale
    scale = float(np.float32(1.0 / 3.0))
    mids = torch.tensor([(grid[c] + grid[c + 1]) / 2 for c in range(0x7E)], dtype=torch.float64)
    centre = (mids * scale).to(in_dtype)
    bits = {torch.float32: torch.int32, torch.float16: torch.int16, torch.bfloat16: torch.int16}[in_dtype]
    around = [centre]
    for d in (-2, -1, 1, 2):  # neighbours in the input dtype (positive values: +1 bit = next representable)
        around.append((centre.view(bits) + d).view(in_dtype))
    stored = torch.cat(around)
    stored = stored[torch.isfinite(stored)]
    _check_quantiser(in_dtype, scale, torch.cat([stored, -stored]))


def _check_quantiser(in_dtype, scale, stored):
    NB, bs, Hkv, D = 8, 16, 1, 128
    n = stored.numel()
    rows = (n + D - 1) // D
    assert rows * 3 <= NB * bs
    xs = torch.zeros(rows * D, dtype=in_dtype)
    xs[:n] = stored
    k = xs.view(rows, 1, D)
    kc = torch.zeros((NB, bs, Hkv, D), dtype=torch.uint8)
    slots = torch.arange(rows, dtype=torch.int64) * 3
    ek, ev = oracle.cache_write(k, k, kc.view(torch.float8_e4m3fn), kc.view(torch.float8_e4m3fn), slots, scale, scale)
    dk = kc.clone().cuda()
    dv = kc.clone().cuda()
    pa.cache_write(k.cuda(), k.cuda(), dk.view(torch.float8_e4m3fn), dv.view(torch.float8_e4m3fn), slots.cuda(),
                   k_scale=scale, v_scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(dk.cpu(), ek.view(torch.uint8)), f"scale {scale}: codes differ from the oracle's"
    assert torch.equal(dv.cpu(), ev.view(torch.uint8))
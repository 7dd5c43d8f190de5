"""The fused decode step (pa_decode_append: the cache write of every
sequence's new token and the decode in one launch) against the two-launch
step it stands for (pa_cache_write then pa_decode) and the oracle.

The fused step reads the new token's rows from k_new / v_new instead of the
slot it writes.  The pools it leaves must be byte-equal to the oracle's cache
write, its output must meet the oracle's tolerances, and it must agree with
the two-launch step to fp32 rounding: the vector-ALU kernel (groups of one or
two heads, fp32 caches) takes the new token first in its item's softmax rather
than last, so its sums run in another order (fp32 outputs within 1e-5, 16-bit
outputs within 1e-5 plus one unit in the last place); the matrix-core kernel
takes it in place, and is bit-exact."""

import pytest
import torch

import paged_kv_cache_447_amd as pa
from pa_workloads import get_config, scaled
from pa_workloads.configs import CONFIG_ORDER
from tests.gpu_common import (TOL_F32, TOL_OUT, gpu_cache_write, gpu_decode, host_inputs, log, max_abs_err,
                              max_err_beyond_rounding, oracle_step, setup)
from tests.test_gpu_parity import SMALL, _bytes

pytestmark = pytest.mark.gpu

# one unit in the last place, relative to the value, and the smallest spacing of each output type
ULP_REL = {"torch.float16": 2.0**-10, "torch.bfloat16": 2.0**-7}
ULP_MIN = {"torch.float16": 2.0**-24, "torch.bfloat16": 2.0**-133}


def fused(cfg, inp, out_dtype=None, partition_size=None, num_workers=0):
    q = inp["q"]
    out = torch.full(q.shape, float("nan"), dtype=out_dtype or q.dtype, device=q.device)
    part = cfg.partition_size if partition_size is None else partition_size
    pa.decode_append(out, q, inp["k_new"], inp["v_new"], inp["k_cache"], inp["v_cache"], inp["slot_mapping"],
                     inp["block_tables"], inp["context_lens"], cfg.block_size, cfg.softmax_scale, cfg.num_kv_heads,
                     partition_size=part, num_workers=num_workers)
    return out


def check(cfg, partition_size=None, num_workers=0, name=""):
    layout, inp = setup(cfg)
    host = host_inputs(inp)
    twin = {k: (v.clone() if torch.is_tensor(v) else v) for k, v in inp.items()}
    # the two-launch step on one copy, the fused step on the other
    gpu_cache_write(cfg, twin)
    want32 = gpu_decode(cfg, twin, out_dtype=torch.float32, partition_size=partition_size, num_workers=num_workers)
    want = gpu_decode(cfg, twin, partition_size=partition_size, num_workers=num_workers)
    got32 = fused(cfg, inp, torch.float32, partition_size, num_workers)
    got = fused(cfg, {**inp, "k_new": inp["k_new"], "v_new": inp["v_new"]}, None, partition_size, num_workers)
    torch.cuda.synchronize()
    ref, kc, vc = oracle_step(cfg, host)
    assert torch.equal(_bytes(inp["k_cache"]), kc.view(torch.uint8)), "k_cache differs from the oracle's write"
    assert torch.equal(_bytes(inp["v_cache"]), vc.view(torch.uint8)), "v_cache differs from the oracle's write"
    d32 = max((got32 - want32).abs().max().item(), 0.0 if got.dtype != torch.float32 else
              (got - want).abs().max().item())
    # outputs in the query's 16-bit type: the roundings of two fp32 values at most 1e-5 apart, so at most
    # 1e-5 plus one unit in the last place apart
    beyond_ulp = 0.0
    if got.dtype != torch.float32:
        w = want.float()
        bound = torch.clamp(w.abs() * ULP_REL[str(got.dtype)], min=ULP_MIN[str(got.dtype)]) + 1e-5
        beyond_ulp = ((got.float() - w).abs() - bound).max().item()
    same = torch.equal(got32.view(torch.int32), want32.view(torch.int32))
    # the query-typed output is held to the bound beyond its own rounding (a correctly rounded bf16 value
    # of magnitude 2-4 is already up to 7.8e-3 from the exact one)
    err, err32 = max_err_beyond_rounding(got, ref), max_abs_err(got32, ref)
    log(f"[{name}] fused vs two-launch: fp32 max|diff|={d32:.3e} (bit-equal: {same}), 16-bit output within "
        f"1e-5 + one ulp: {beyond_ulp <= 0}; vs oracle: beyond output rounding {err:.3e}, err32={err32:.3e}")
    assert d32 <= 1e-5, "fp32 output differs from the two-launch step beyond rounding"
    if cfg.num_heads // cfg.num_kv_heads >= 4 and cfg.kv_dtype in ("f16", "bf16"):  # the matrix-core kernel
        assert same and torch.equal(got.view(torch.uint8), want.view(torch.uint8)), \
            "the matrix-core fused step differs from the two-launch step"
    assert beyond_ulp <= 0, "16-bit output differs from the two-launch step by more than one unit in the last place"
    assert err <= TOL_OUT[cfg.kv_dtype] and err32 <= TOL_F32[cfg.kv_dtype]


@pytest.mark.parametrize("name", [n for n in CONFIG_ORDER if get_config(n).kv_dtype != "fp8"])
def test_full_size_fused_step(name):
    check(get_config(name), name=name)


@pytest.mark.parametrize("case", sorted(k for k, c in SMALL.items() if c.kv_dtype != "fp8"))
@pytest.mark.parametrize("split", [(0, 0), (64, 0), (0, 4), (16, 100)], ids=["p0w0", "p64w0", "p0w4", "p16w100"])
def test_small_fused_steps(case, split):
    cfg = SMALL[case]
    part, workers = split
    part = part if part % cfg.block_size == 0 else 0
    check(cfg, partition_size=part, num_workers=workers, name=f"{case} p={part} w={workers}")


# Context lengths at the edges of the new token's handling: a sequence whose only token is the new one;
# new tokens that open a work unit of their own at partition sizes 16 and 32 (lengths 16 k + 1), so that
# the last segment holds no paged token; new tokens that close a unit (16 k, 32 k); short and longer rest.
EDGE_LENS = (1, 2, 15, 16, 17, 31, 32, 33, 48, 49, 64, 65, 1, 97, 129, 3)
EDGES = {
    "mha_f16": scaled(get_config("llama7b"), num_seqs=len(EDGE_LENS), num_heads=4, num_kv_heads=4,
                      ctx_kind="fixed", ctx_fixed=EDGE_LENS, num_blocks=300, max_blocks_per_seq=12),
    "gqa2_bf16_d64": scaled(get_config("llama7b"), num_seqs=len(EDGE_LENS), num_heads=8, num_kv_heads=4,
                            head_dim=64, q_dtype="bf16", kv_dtype="bf16", ctx_kind="fixed", ctx_fixed=EDGE_LENS,
                            num_blocks=300, max_blocks_per_seq=12),
    "mha_f32_bs32": scaled(get_config("tiny"), num_seqs=len(EDGE_LENS), num_heads=2, num_kv_heads=2, head_dim=128,
                           block_size=32, ctx_fixed=EDGE_LENS, num_blocks=200, max_blocks_per_seq=6),
    "gqa8_f16": scaled(get_config("gqa70b"), num_seqs=len(EDGE_LENS), num_heads=16, num_kv_heads=2,
                       ctx_kind="fixed", ctx_fixed=EDGE_LENS, num_blocks=300, max_blocks_per_seq=6,
                       allocator="shuffled"),
}


@pytest.mark.parametrize("case", sorted(EDGES))
@pytest.mark.parametrize("split", [(0, 0), (16, 0), (32, 5), (16, 200)], ids=["p0w0", "p16w0", "p32w5", "p16w200"])
def test_fused_step_new_token_edges(case, split):
    cfg = EDGES[case]
    part, workers = split
    part = part if part % cfg.block_size == 0 else 0
    check(cfg, partition_size=part, num_workers=workers, name=f"edges {case} p={part} w={workers}")


def test_fused_step_refuses_fp8():
    cfg = scaled(get_config("fp8_long"), num_seqs=2, num_blocks=600, max_blocks_per_seq=256, ctx_lo=100, ctx_hi=400)
    layout, inp = setup(cfg)
    with pytest.raises(pa.PaError) as e:
        fused(cfg, inp)
    assert e.value.status == -5


def test_fused_step_replays_in_a_graph():
    """The fused step captured in a HIP graph (torch.cuda.graph) and replayed:
    every replay equals the eager call bit for bit, with eager calls and a
    changed query between replays."""
    cfg = SMALL["gqa8_f16"]
    for c in (cfg, SMALL["mha_f16_edges"]):
        layout, inp = setup(c)
        ws = pa.new_workspace(inp["q"], c.num_kv_heads)
        out = torch.empty_like(inp["q"])
        q_a = inp["q"].clone()
        q_b = torch.randn_like(q_a)

        def step(o):
            pa.decode_append(o, inp["q"], inp["k_new"], inp["v_new"], inp["k_cache"], inp["v_cache"],
                             inp["slot_mapping"], inp["block_tables"], inp["context_lens"], c.block_size,
                             c.softmax_scale, c.num_kv_heads, workspace=ws)
            return o

        refs = {}
        for name, qv in (("a", q_a), ("b", q_b)):
            inp["q"].copy_(qv)
            refs[name] = step(torch.empty_like(out)).clone()
        torch.cuda.synchronize()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            step(out)  # warm-up on the capture stream
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(out)
        for r in range(4):
            name = "a" if r % 2 == 0 else "b"
            inp["q"].copy_(q_a if name == "a" else q_b)
            out.fill_(float("nan"))
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, refs[name]), f"replay {r} differs from the eager call"
            eager = step(torch.empty_like(out))
            torch.cuda.synchronize()
            assert torch.equal(eager, refs[name])
        log(f"[graph fused step G={c.num_heads // c.num_kv_heads}] 4 replays bit-identical to the eager call")

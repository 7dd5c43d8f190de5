"""Paged decode (and prefill) benchmark on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config NAME] [--also NAMES] [--no-cpu-baseline]

A step is one pass of the whole hot path over one batch: the cache write of
each sequence's new token, then paged decode (balanced split-context workers
with the log-sum-exp merge in the same kernel) over the workload's context
lengths.  For 16-bit and fp32 caches the step is one pa_decode_append launch
(the cache write fused into the decode); for fp8 caches it is pa_cache_write
then pa_decode.  Inputs are resident in HBM before timing starts; steps rotate
over several independent input sets so that consecutive steps do not hit in
the 256 MB Infinity Cache.

With a prefill workload as --config (prefill_7b, verify_gqa70b, prefill_small)
a step is instead the cache write of every new token of the step followed by
pa_prefill over all query rows, and the line reports attention TFLOP/s.  With
a block-copy workload (cow_llama7b, swap_out_gqa70b, swap_in_gqa70b) a step is
one pa_copy_blocks launch, and the line reports bytes moved per second.  With
a multi-layer workload (llama7b_x8, gqa70b_x8) a step writes every layer's new
token (one cache-write launch over the flattened pools) and decodes all layers
in one pa_decode_layers launch; the line reports K/V GB/s like decode.

Prints ONE JSON line: effective KV bandwidth (logical K/V bytes of every valid
token per step / step time) in GB/s, tokens/s, the main kernel's roofline
position (its launches timed back to back between two HIP events on its
stream; HBM traffic from the committed rocprofv3 counter summary while the
kernel sources match it), the same figures for the --also workloads (default
gqa70b), and the fp64 CPU oracle's throughput on a sample of the same workload
on all host threads and on one, as a reported baseline.

--copy-calibration adds a plain device-to-device copy of known size after the
timed region, so that a rocprofv3 counter run of this command also measures
what FETCH_SIZE / WRITE_SIZE read for a known number of bytes.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

METRIC = "paged decode effective KV HBM GB/s (% of MI355X peak) and tokens/s at 1 GPU"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E peak, GB/s


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--config", default="llama7b")
    ap.add_argument("--partition-size", type=int, default=-1, help="-1: the workload's own setting")
    ap.add_argument("--num-workers", type=int, default=0, help="0: the library's choice")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target wall time of the oracle sample")
    ap.add_argument("--also", default="gqa70b",
                    help="comma-separated decode workloads also timed (step and kernel) in the same run; '' for none")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 512 MiB device copy (reference for hardware byte counters)")
    ap.add_argument("--no-read-ceiling", action="store_true",
                    help="skip the streaming-read ceiling measured after the decode legs")
    return ap.parse_args()


ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {
    "decode": ["pa_sched.h", "pa_device.h", "pa_internal.h", "mfma_core.h", "decode_valu.hip", "decode_mfma.hip"],
    "prefill": ["pa_device.h", "pa_internal.h", "mfma_core.h", "prefill_mfma.hip"],
    "blocks": ["pa_device.h", "pa_internal.h", "block_copy.hip"],
}
HOST_LINK_PEAK_GBS = 64.0  # PCIe 5.0 x16, one direction, GB/s
MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 / bf16 matrix peak, TFLOP/s


def kernel_source_hash(kind: str = "decode") -> str:
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "paged_kv_cache_447_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kind: str = "decode"):
    """HBM bytes per launch of the workload's main kernel from the committed
    counter summary, or None if there is none for this workload or the kernel
    sources changed since."""
    try:
        with open(TRAFFIC) as f:
            rec = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != kernel_source_hash(kind):
        return None
    return rec.get("bytes_per_launch")


def back_to_back_ms(fn, sets, steps, stream) -> float:
    """Milliseconds per call of fn over `steps` calls issued back to back on
    `stream` (rotating over the input sets), bracketed by two HIP events on that
    stream: the launches' own time, with no gaps from event records between them."""
    import torch

    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(steps):
        fn(sets[i % len(sets)])
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


READ_CEILING_BYTES = 4 << 30  # 16x the 256 MB last-level cache
READ_CEILING_GRIDS = (1024, 2048, 4096, 8192, 16384)


def read_ceiling(dev, steps: int = 10) -> dict:
    """The part's practical streaming-read rate: pa_stream_read over a 4 GiB
    buffer of seeded random words, at five grid sizes x 1, 4 or 8 loads in
    flight x ordinary or non-temporal loads, each shape timed by HIP events
    around `steps` launches back to back on one stream.  Every shape's checksum
    (the XOR of its partials) must equal a separate XOR fold of the buffer."""
    import numpy as np
    import torch

    import paged_kv_cache_447_amd as pa

    stream = torch.cuda.current_stream(dev)
    gen = torch.Generator(device=dev).manual_seed(1234)
    buf = torch.empty(READ_CEILING_BYTES // 4, dtype=torch.int32, device=dev).random_(generator=gen)
    fold = buf
    while fold.numel() > 1:  # the element count is a power of two
        h = fold.numel() // 2
        fold = torch.bitwise_xor(fold[:h], fold[h:])
    want = int(fold.item()) & 0xFFFFFFFF
    del fold
    partials = torch.zeros(max(READ_CEILING_GRIDS), dtype=torch.int32, device=dev)
    best = {}
    for nt in (False, True):
        for loads in (1, 4, 8):
            for grid in READ_CEILING_GRIDS:
                def run(_, grid=grid, loads=loads, nt=nt):
                    pa.stream_read(buf, partials, grid, loads, nt, stream=stream.cuda_stream)

                run(None)
                torch.cuda.synchronize()
                got = int(np.bitwise_xor.reduce(partials[:grid].cpu().numpy().view(np.uint32)))
                if got != want:
                    raise RuntimeError(f"pa_stream_read checksum {got:#x} != {want:#x} "
                                       f"(grid {grid}, {loads} loads, nontemporal={nt})")
                gbs = READ_CEILING_BYTES / (back_to_back_ms(run, [None], steps, stream) * 1e-3) / 1e9
                key = ("nontemporal" if nt else "ordinary", loads)
                if key not in best or gbs > best[key][0]:
                    best[key] = (gbs, grid)
    del buf, partials
    torch.cuda.empty_cache()
    top_key = max(best, key=lambda k: best[k][0])
    top_gbs, top_grid = best[top_key]
    return {
        "GB/s": round(top_gbs, 1),
        "frac_of_peak": round(top_gbs / HBM_PEAK_GBS, 4),
        "loads": top_key[0],
        "loads_in_flight": top_key[1],
        "workgroups": top_grid,
        "bytes": READ_CEILING_BYTES,
        "launches_per_shape": steps,
        "best_per_kind": {f"{k[0]}_x{k[1]}": {"GB/s": round(v[0], 1), "workgroups": v[1]}
                          for k, v in sorted(best.items())},
        "kernel": "pa_stream_read (grid-stride 16-byte loads folded into an XOR checksum)",
    }


def oracle_rate(run_once, seconds: float):
    """(repetitions, wall seconds) of run_once() repeated for about `seconds`."""
    reps, t_start = 0, time.perf_counter()
    while True:
        run_once()
        reps += 1
        el = time.perf_counter() - t_start
        if el >= seconds or reps >= 1000:
            return reps, el


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        sys.stderr.write("bench.py measures one GPU: this build has no multi-GPU path "
                         "(decode shards by sequence or kv head with no exchange); run with --gpus 1\n")
        sys.exit(2)

    import numpy as np
    import torch

    import paged_kv_cache_447_amd as pa
    from pa_workloads import algorithmic_bytes, get_config, kv_bytes, make_inputs, make_layout

    if not torch.cuda.is_available():
        sys.stderr.write("bench.py needs a GPU\n")
        sys.exit(1)
    pa.load_library()  # fails loudly if libpa.so is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    from pa_workloads.prefill import PREFILL_CONFIGS

    if args.config in PREFILL_CONFIGS:
        print(json.dumps(bench_prefill(args, PREFILL_CONFIGS[args.config], dev)), flush=True)
        return
    from pa_workloads.layers import LAYER_CONFIGS

    if args.config in LAYER_CONFIGS:
        print(json.dumps(bench_layers(args, LAYER_CONFIGS[args.config], dev)), flush=True)
        return
    from pa_workloads.blocks import BLOCK_CONFIGS

    if args.config in BLOCK_CONFIGS:
        print(json.dumps(bench_blocks(args, BLOCK_CONFIGS[args.config], dev)), flush=True)
        return

    cfg = get_config(args.config)
    part = cfg.partition_size if args.partition_size < 0 else args.partition_size
    layout = make_layout(cfg)
    ctx = layout.context_lens
    step_kv = kv_bytes(cfg, ctx)
    step_alg = algorithmic_bytes(cfg, ctx)
    pool_bytes = 2 * cfg.num_blocks * cfg.block_size * cfg.num_kv_heads * cfg.head_dim * \
        {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1}[cfg.kv_dtype]
    nsets = max(2, math.ceil(1e9 / max(1, step_kv)))
    nsets = min(nsets, max(2, int(40e9 // pool_bytes)))
    sets = []
    for i in range(nsets):
        inp = make_inputs(cfg, layout, dev, seed_offset=i)
        inp["out"] = torch.zeros_like(inp["q"])  # sets that a short run never reaches stay finite
        inp["ws"] = pa.new_workspace(inp["q"], cfg.num_kv_heads, args.num_workers)
        sets.append(inp)
    host0 = None
    if not args.no_cpu_baseline:  # generator bytes of set 0, before any kernel touches them
        host0 = {k: (v.cpu() if torch.is_tensor(v) else v) for k, v in sets[0].items() if k not in ("out", "ws")}
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream

    fused = cfg.kv_dtype != "fp8"  # one launch per step; fp8 caches write the new rows with pa_cache_write

    def write(inp):
        pa.cache_write(inp["k_new"], inp["v_new"], inp["k_cache"], inp["v_cache"], inp["slot_mapping"],
                       k_scale=inp["k_scale"], v_scale=inp["v_scale"], stream=sptr)

    def decode(inp):
        pa.decode(inp["out"], inp["q"], inp["k_cache"], inp["v_cache"], inp["block_tables"], inp["context_lens"],
                  cfg.block_size, cfg.softmax_scale, cfg.num_kv_heads, k_scale=inp["k_scale"],
                  v_scale=inp["v_scale"], partition_size=part, num_workers=args.num_workers, workspace=inp["ws"],
                  stream=sptr)

    def append(inp):
        pa.decode_append(inp["out"], inp["q"], inp["k_new"], inp["v_new"], inp["k_cache"], inp["v_cache"],
                         inp["slot_mapping"], inp["block_tables"], inp["context_lens"], cfg.block_size,
                         cfg.softmax_scale, cfg.num_kv_heads, partition_size=part, num_workers=args.num_workers,
                         workspace=inp["ws"], stream=sptr)

    def step(inp):
        if fused:
            append(inp)
        else:
            write(inp)
            decode(inp)

    for i in range(args.warmup):
        step(sets[i % nsets])
    torch.cuda.synchronize()

    # timed region 1: whole steps back to back
    ms_per_step = back_to_back_ms(step, sets, args.steps, stream)
    # timed region 2: the step's main kernel alone, back to back (the fused
    # launch, or the decode launch of a two-launch step)
    kernel_ms = back_to_back_ms(append if fused else decode, sets, args.steps, stream)
    # the two-launch form of the same step, for comparison
    two_launch_ms = back_to_back_ms(lambda inp: (write(inp), decode(inp)), sets, args.steps, stream) if fused else None
    for inp in sets:
        if not torch.isfinite(inp["out"]).all():
            raise RuntimeError("non-finite decode output")

    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float16, device=dev).fill_(1.0)  # 512 MiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # the fused launch also writes every sequence's new K and V rows (and reads its slot)
    kernel_alg = step_alg + (new_row_bytes(cfg) + 8 * cfg.num_seqs if fused else 0)
    achieved = kernel_alg / (kernel_ms * 1e-3) / 1e9
    value = step_kv / (ms_per_step * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "f16": "f16", "bf16": "bf16", "fp8": "fp8-e4m3 kv / f16"}[cfg.kv_dtype],
        "data": "synthetic (seeded N(0,1) values, seeded block allocator)",
        "config": {
            "workload": cfg.name,
            "num_seqs": cfg.num_seqs,
            "num_heads": cfg.num_heads,
            "num_kv_heads": cfg.num_kv_heads,
            "head_dim": cfg.head_dim,
            "block_size": cfg.block_size,
            "kv_dtype": cfg.kv_dtype,
            "mean_context": float(np.mean(ctx)),
            "partition_size": part,
            "num_workers": pa.num_workers(args.num_workers),
            "input_sets": nsets,
            "kv_bytes_per_step": step_kv,
            "step": "pa_decode_append (cache write + decode, one launch)" if fused
                    else "pa_cache_write + pa_decode (two launches)",
            **({"fp8_scales": f"one per {cfg.fp8_scales}"} if cfg.kv_dtype == "fp8" else {}),
        },
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(cfg.num_seqs / (ms_per_step * 1e-3), 1),
        "roofline": {
            "kernel": ("fused step: new-row cache write + " if fused else "") +
                      "decode (paged K/V gather + QK + online softmax + PV + in-kernel log-sum-exp merge)",
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(cfg.name),
            "kernel_ms": round(kernel_ms, 5),
            "timing": "HIP events around the kernel alone launched back to back on its stream",
            "algorithmic_bytes_per_launch": kernel_alg,
        },
        "two_launch_ms_per_step": round(two_launch_ms, 5) if two_launch_ms else None,
        "cpu_baseline": None,
    }
    if args.also:
        result["also"] = {name: also_decode(args, name, dev) for name in args.also.split(",")
                          if name and name != cfg.name}
    if not args.no_read_ceiling:
        rc = read_ceiling(dev)
        result["read_ceiling"] = rc
        result["roofline"]["frac_of_read_ceiling"] = round(achieved / rc["GB/s"], 4)
        for leg in result.get("also", {}).values():
            leg["frac_of_read_ceiling"] = round(leg["roofline_frac"] * HBM_PEAK_GBS / rc["GB/s"], 4)

    if host0 is not None:
        import oracle

        cores = len(os.sched_getaffinity(0))
        nthreads = max(1, min(cores, 64))
        kc, vc = oracle.cache_write(host0["k_new"], host0["v_new"], host0["k_cache"], host0["v_cache"],
                                    host0["slot_mapping"], host0["k_scale"], host0["v_scale"], inplace=True)

        def oracle_step(nt):
            def run():
                oracle.cache_write(host0["k_new"], host0["v_new"], kc, vc, host0["slot_mapping"], host0["k_scale"],
                                   host0["v_scale"], inplace=True)
                oracle.paged_decode(host0["q"], kc, vc, host0["block_tables"], host0["context_lens"],
                                    cfg.softmax_scale, cfg.num_kv_heads, host0["k_scale"], host0["v_scale"],
                                    nthreads=nt)
            return run

        reps, el = oracle_rate(oracle_step(nthreads), args.cpu_seconds)
        reps1, el1 = oracle_rate(oracle_step(1), args.cpu_seconds)
        result["cpu_baseline"] = {
            "value": round(step_kv * reps / el / 1e9, 4),
            "unit": "GB/s",
            "cores": nthreads,
            "kind": "oracle",
            "sample": f"{reps} full {cfg.name} steps (cache write + fp64 decode of all {cfg.num_seqs} sequences), "
                      f"{el:.1f} s wall, {nthreads} threads",
            "tokens_per_s": round(cfg.num_seqs * reps / el, 2),
            "single_thread": {
                "value": round(step_kv * reps1 / el1 / 1e9, 4),
                "unit": "GB/s",
                "cores": 1,
                "sample": f"{reps1} full {cfg.name} steps, {el1:.1f} s wall, 1 thread",
                "tokens_per_s": round(cfg.num_seqs * reps1 / el1, 2),
            },
        }
    print(json.dumps(result), flush=True)


def new_row_bytes(cfg) -> int:
    """Bytes of the new K and V rows a step writes (one token per sequence)."""
    return 2 * cfg.num_seqs * cfg.num_kv_heads * cfg.head_dim * {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1}[cfg.kv_dtype]


def also_decode(args, name: str, dev) -> dict:
    """A second decode workload's step and kernel time on the same box (no
    oracle): the fused step for 16-bit caches, the two-launch step for fp8."""
    import numpy as np
    import torch

    import paged_kv_cache_447_amd as pa
    from pa_workloads import algorithmic_bytes, get_config, kv_bytes, make_inputs, make_layout

    cfg = get_config(name)
    layout = make_layout(cfg)
    ctx = layout.context_lens
    step_kv, step_alg = kv_bytes(cfg, ctx), algorithmic_bytes(cfg, ctx)
    pool_bytes = 2 * cfg.num_blocks * cfg.block_size * cfg.num_kv_heads * cfg.head_dim * \
        {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1}[cfg.kv_dtype]
    nsets = min(max(2, math.ceil(1e9 / max(1, step_kv))), max(2, int(40e9 // pool_bytes)))
    sets = []
    for i in range(nsets):
        inp = make_inputs(cfg, layout, dev, seed_offset=i)
        inp["out"] = torch.zeros_like(inp["q"])
        inp["ws"] = pa.new_workspace(inp["q"], cfg.num_kv_heads)
        sets.append(inp)
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream
    fused = cfg.kv_dtype != "fp8"

    def decode(inp):
        pa.decode(inp["out"], inp["q"], inp["k_cache"], inp["v_cache"], inp["block_tables"], inp["context_lens"],
                  cfg.block_size, cfg.softmax_scale, cfg.num_kv_heads, k_scale=inp["k_scale"],
                  v_scale=inp["v_scale"], partition_size=cfg.partition_size, workspace=inp["ws"], stream=sptr)

    def step(inp):
        if fused:
            pa.decode_append(inp["out"], inp["q"], inp["k_new"], inp["v_new"], inp["k_cache"], inp["v_cache"],
                             inp["slot_mapping"], inp["block_tables"], inp["context_lens"], cfg.block_size,
                             cfg.softmax_scale, cfg.num_kv_heads, partition_size=cfg.partition_size,
                             workspace=inp["ws"], stream=sptr)
        else:
            pa.cache_write(inp["k_new"], inp["v_new"], inp["k_cache"], inp["v_cache"], inp["slot_mapping"],
                           k_scale=inp["k_scale"], v_scale=inp["v_scale"], stream=sptr)
            decode(inp)

    for i in range(max(10, args.warmup // 2)):
        step(sets[i % nsets])
    steps = max(50, args.steps // 2)
    ms_step = back_to_back_ms(step, sets, steps, stream)
    ms_kernel = back_to_back_ms(step if fused else decode, sets, steps, stream)
    kernel_alg = step_alg + (new_row_bytes(cfg) + 8 * cfg.num_seqs if fused else 0)
    del sets
    torch.cuda.empty_cache()
    return {
        "ms_per_step": round(ms_step, 5),
        "kv_gb_per_s": round(step_kv / (ms_step * 1e-3) / 1e9, 2),
        "pct_of_hbm_peak": round(100.0 * step_kv / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
        "kernel_ms": round(ms_kernel, 5),
        "roofline_frac": round(kernel_alg / (ms_kernel * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "algorithmic_bytes_per_launch": kernel_alg,
        "steps": steps,
        "step": "pa_decode_append" if fused else "pa_cache_write + pa_decode",
    }


def bench_prefill(args, pcfg, dev) -> dict:
    """One step = cache write of the step's new K/V rows, then pa_prefill over
    every query row.  Same protocol as decode: rotating input sets, warmup,
    whole steps timed back to back, then HIP events around the prefill launch."""
    import numpy as np
    import torch

    import paged_kv_cache_447_amd as pa
    from pa_workloads.generate import ELEM_BYTES
    from pa_workloads.prefill import (make_prefill_inputs, make_prefill_layout, prefill_algorithmic_bytes,
                                      prefill_flops, prefill_kv_bytes)

    cfg = pcfg.base
    pl = make_prefill_layout(pcfg)
    ctx = pl.layout.context_lens
    N = int(pl.query_start_loc[-1])
    flops = prefill_flops(pcfg, pl)
    kvb = prefill_kv_bytes(pcfg, pl)
    alg_bytes = prefill_algorithmic_bytes(pcfg, pl)
    pool_bytes = 2 * cfg.num_blocks * cfg.block_size * cfg.num_kv_heads * cfg.head_dim * ELEM_BYTES[cfg.kv_dtype]
    nsets = max(2, math.ceil(1e9 / max(1, kvb)))
    nsets = min(nsets, max(2, int(40e9 // pool_bytes)))
    sets = []
    for i in range(nsets):
        inp = make_prefill_inputs(pcfg, pl, dev, seed_offset=i)
        inp["out"] = torch.zeros_like(inp["q"])  # sets that a short run never reaches stay finite
        inp["ws"] = pa.new_prefill_workspace(dev)
        sets.append(inp)
    host0 = None
    if not args.no_cpu_baseline:
        host0 = {k: (v.cpu() if torch.is_tensor(v) else v) for k, v in sets[0].items() if k not in ("out", "ws")}
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream

    def write(inp):
        pa.cache_write(inp["k_new"], inp["v_new"], inp["k_cache"], inp["v_cache"], inp["slot_mapping"],
                       k_scale=inp["k_scale"], v_scale=inp["v_scale"], stream=sptr)

    def prefill(inp):
        pa.prefill(inp["out"], inp["q"], inp["k_cache"], inp["v_cache"], inp["block_tables"], inp["context_lens"],
                   inp["query_start_loc"], cfg.block_size, cfg.softmax_scale, cfg.num_kv_heads,
                   k_scale=inp["k_scale"], v_scale=inp["v_scale"], workspace=inp["ws"], stream=sptr)

    for i in range(args.warmup):
        write(sets[i % nsets])
        prefill(sets[i % nsets])
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(args.steps):
        write(sets[i % nsets])
        prefill(sets[i % nsets])
    t1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps
    # the prefill kernel alone, back to back (the cache already holds the step's rows)
    kernel_ms = back_to_back_ms(prefill, sets, args.steps, stream)
    for inp in sets:
        if not torch.isfinite(inp["out"]).all():
            raise RuntimeError("non-finite prefill output")
    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float16, device=dev).fill_(1.0)  # 512 MiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    ridge = MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    mfma_bound = flops / alg_bytes >= ridge
    tflops = flops / (kernel_ms * 1e-3) / 1e12
    gbs = alg_bytes / (kernel_ms * 1e-3) / 1e9
    value = flops / (ms_per_step * 1e-3) / 1e12
    if mfma_bound:
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tflops / MFMA_PEAK_TFLOPS, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4)}
    roof.update({
        "traffic": measured_traffic(cfg.name, "prefill"),
        "kernel": "prefill (paged K/V gather + causal QK + online softmax + PV)",
        "kernel_ms": round(kernel_ms, 5),
        "algorithmic_flops_per_launch": flops,
        "algorithmic_bytes_per_launch": alg_bytes,
        "flops_per_byte": round(flops / alg_bytes, 2),
    })
    result = {
        "metric": "paged prefill attention TFLOP/s (causal flops per step / step time) at 1 GPU",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.kv_dtype,
        "data": "synthetic (seeded N(0,1) values, seeded block allocator)",
        "config": {
            "workload": cfg.name,
            "num_seqs": cfg.num_seqs,
            "query_rows": N,
            "num_heads": cfg.num_heads,
            "num_kv_heads": cfg.num_kv_heads,
            "head_dim": cfg.head_dim,
            "block_size": cfg.block_size,
            "kv_dtype": cfg.kv_dtype,
            "mean_context": float(np.mean(ctx)),
            "input_sets": nsets,
        },
        "query_tokens_per_s": round(N / (ms_per_step * 1e-3), 1),
        "kv_gb_per_s": round(kvb / (ms_per_step * 1e-3) / 1e9, 2),
        "roofline": roof,
        "cpu_baseline": None,
    }
    if host0 is not None:
        import oracle

        cores = len(os.sched_getaffinity(0))
        nthreads = max(1, min(cores, 64))
        kc, vc = oracle.cache_write(host0["k_new"], host0["v_new"], host0["k_cache"], host0["v_cache"],
                                    host0["slot_mapping"], host0["k_scale"], host0["v_scale"], inplace=True)
        # the sample: the step's first sequence (all of its query rows), repeated
        qsl = host0["query_start_loc"]
        n0 = int(qsl[1])
        q0 = host0["q"][:n0].contiguous()
        sub_flops = 4 * cfg.head_dim * cfg.num_heads * (n0 * (int(ctx[0]) - n0) + n0 * (n0 + 1) // 2)
        reps, t_start = 0, time.perf_counter()
        while True:
            oracle.paged_prefill(q0, kc, vc, host0["block_tables"][:1], host0["context_lens"][:1],
                                 qsl[:2].contiguous(), cfg.softmax_scale, cfg.num_kv_heads, host0["k_scale"],
                                 host0["v_scale"], nthreads=nthreads)
            reps += 1
            el = time.perf_counter() - t_start
            if el >= args.cpu_seconds or reps >= 1000:
                break
        result["cpu_baseline"] = {
            "value": round(sub_flops * reps / el / 1e12, 6),
            "unit": "TFLOP/s",
            "cores": nthreads,
            "kind": "oracle",
            "sample": f"{reps} x the fp64 prefill of sequence 0 of {cfg.name} ({n0} query rows, context "
                      f"{int(ctx[0])}, all {cfg.num_heads} heads), {el:.1f} s wall, {nthreads} threads",
        }
    return result


def bench_layers(args, lcfg, dev) -> dict:
    """Decode of L layers sharing one layout: one step = the cache write of all
    layers' new tokens plus one pa_decode_layers launch."""
    import numpy as np
    import torch

    import paged_kv_cache_447_amd as pa
    from pa_workloads import algorithmic_bytes, kv_bytes, make_layout
    from pa_workloads.layers import flat_slots, make_layer_inputs

    cfg = lcfg.base
    L = lcfg.num_layers
    layout = make_layout(cfg)
    ctx = layout.context_lens
    step_kv = L * kv_bytes(cfg, ctx)
    step_alg = L * algorithmic_bytes(cfg, ctx)
    nsets = 2
    sets = []
    for i in range(nsets):
        inp = make_layer_inputs(lcfg, layout, dev, seed_offset=i)
        inp["out"] = torch.zeros_like(inp["q"])
        inp["ws"] = pa.new_workspace(inp["q"], cfg.num_kv_heads)
        NB = cfg.num_blocks
        inp["kc_flat"] = inp["k_cache"].view((L * NB,) + tuple(inp["k_cache"].shape[2:]))
        inp["vc_flat"] = inp["v_cache"].view((L * NB,) + tuple(inp["v_cache"].shape[2:]))
        inp["kn_flat"] = inp["k_new"].reshape((-1,) + tuple(inp["k_new"].shape[2:]))
        inp["vn_flat"] = inp["v_new"].reshape((-1,) + tuple(inp["v_new"].shape[2:]))
        inp["slots_flat"] = flat_slots(inp["slot_mapping"], L, NB * cfg.block_size)
        sets.append(inp)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream

    def write(inp):
        pa.cache_write(inp["kn_flat"], inp["vn_flat"], inp["kc_flat"], inp["vc_flat"], inp["slots_flat"],
                       k_scale=inp["k_scale"], v_scale=inp["v_scale"], stream=sptr)

    def decode(inp):
        pa.decode_layers(inp["out"], inp["q"], inp["k_cache"], inp["v_cache"], inp["block_tables"],
                         inp["context_lens"], cfg.block_size, cfg.softmax_scale, cfg.num_kv_heads,
                         k_scale=inp["k_scale"], v_scale=inp["v_scale"], workspace=inp["ws"], stream=sptr)

    for i in range(args.warmup):
        write(sets[i % nsets])
        decode(sets[i % nsets])
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(args.steps):
        write(sets[i % nsets])
        decode(sets[i % nsets])
    t1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps
    # the multi-layer decode kernel alone, back to back
    kernel_ms = back_to_back_ms(decode, sets, args.steps, stream)
    for inp in sets:
        if not torch.isfinite(inp["out"]).all():
            raise RuntimeError("non-finite decode output")
    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float16, device=dev).fill_(1.0)  # 512 MiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    achieved = step_alg / (kernel_ms * 1e-3) / 1e9
    value = step_kv / (ms_per_step * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.kv_dtype,
        "data": "synthetic (seeded N(0,1) values, seeded block allocator)",
        "config": {"workload": lcfg.name, "layers": L, "num_seqs": cfg.num_seqs, "num_heads": cfg.num_heads,
                   "num_kv_heads": cfg.num_kv_heads, "head_dim": cfg.head_dim, "block_size": cfg.block_size,
                   "kv_dtype": cfg.kv_dtype, "mean_context": float(np.mean(ctx)), "input_sets": nsets,
                   "kv_bytes_per_step": step_kv},
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(cfg.num_seqs / (ms_per_step * 1e-3), 1),
        "roofline": {"kernel": "decode_layers (paged decode of all layers in one launch)", "bound": "hbm",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(lcfg.name), "kernel_ms": round(kernel_ms, 5),
                     "algorithmic_bytes_per_launch": step_alg},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        import oracle

        cores = len(os.sched_getaffinity(0))
        nthreads = max(1, min(cores, 64))
        h = {k: sets[0][k][0].cpu() for k in ("q", "k_cache", "v_cache")}
        bt, cl = sets[0]["block_tables"].cpu(), sets[0]["context_lens"].cpu()
        reps, t_start = 0, time.perf_counter()
        while True:
            oracle.paged_decode(h["q"], h["k_cache"], h["v_cache"], bt, cl, cfg.softmax_scale, cfg.num_kv_heads,
                                nthreads=nthreads)
            reps += 1
            el = time.perf_counter() - t_start
            if el >= args.cpu_seconds or reps >= 1000:
                break
        result["cpu_baseline"] = {
            "value": round(kv_bytes(cfg, ctx) * reps / el / 1e9, 4),
            "unit": "GB/s",
            "cores": nthreads,
            "kind": "oracle",
            "sample": f"{reps} fp64 decodes of layer 0 of {lcfg.name} (all {cfg.num_seqs} sequences), "
                      f"{el:.1f} s wall, {nthreads} threads",
        }
    if not args.no_read_ceiling:
        del sets
        torch.cuda.empty_cache()
        rc = read_ceiling(dev)
        result["read_ceiling"] = rc
        result["roofline"]["frac_of_read_ceiling"] = round(achieved / rc["GB/s"], 4)
    return result


def bench_blocks(args, cfg, dev) -> dict:
    """One step = one pa_copy_blocks launch over the workload's pairs, rotating
    over independent pool sets, timed back to back."""
    import numpy as np
    import torch

    import paged_kv_cache_447_amd as pa
    from pa_workloads.blocks import block_mapping, pool_shapes, random_pool

    src_shape, dst_shape, src_host, dst_host = pool_shapes(cfg)
    m = torch.from_numpy(block_mapping(cfg)).to(dev)
    dt = cfg.base.kv_dtype
    moved = cfg.bytes_moved()  # K and V, read + written
    nsets = 2
    sets = []
    for i in range(nsets):
        base = 1000 * cfg.seed + 10 * i
        sk = random_pool(src_shape, dt, base + 1, dev, pin=src_host)
        sv = random_pool(src_shape, dt, base + 2, dev, pin=src_host)
        if cfg.kind == "cow":
            dk, dv = sk, sv
        else:
            dk = random_pool(dst_shape, dt, base + 3, dev, pin=dst_host)
            dv = random_pool(dst_shape, dt, base + 4, dev, pin=dst_host)
        sets.append((dk, dv, sk, sv))
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream

    def step(i):
        dk, dv, sk, sv = sets[i % nsets]
        pa.copy_blocks(dk, dv, sk, sv, m, stream=sptr)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(args.steps):
        step(i)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps
    kernel_ms = ms_per_step  # a step is the one copy launch, timed back to back above
    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float16, device=dev).fill_(1.0)  # 512 MiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    value = moved / (ms_per_step * 1e-3) / 1e9
    if cfg.kind == "cow":
        ach = moved / (kernel_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "algorithmic_bytes_per_launch": moved}
    else:
        link = moved // 2  # the bytes that cross the host link, in one direction
        ach = link / (kernel_ms * 1e-3) / 1e9
        roof = {"bound": "host-link", "achieved": round(ach, 2), "peak": HOST_LINK_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HOST_LINK_PEAK_GBS, 4), "algorithmic_bytes_per_launch": link}
    roof.update({"traffic": measured_traffic(cfg.name, "blocks") if cfg.kind == "cow" else None,
                 "kernel": "copy_blocks (whole-block gather/scatter by a block mapping)",
                 "kernel_ms": round(kernel_ms, 5)})
    result = {
        "metric": "paged block copy GB/s (K and V bytes read + written per step / step time) at 1 GPU",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u8",
        "data": "synthetic (seeded pools and block mapping)",
        "config": {"workload": cfg.name, "kind": cfg.kind, "num_pairs": cfg.num_pairs,
                   "block_bytes": cfg.block_bytes, "kv_dtype": dt, "device_blocks": cfg.base.num_blocks,
                   "input_sets": nsets},
        "roofline": roof,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        import oracle

        dk, dv, sk, sv = sets[0]
        hs_k, hs_v = sk.cpu(), sv.cpu()
        hd_k = hs_k if cfg.kind == "cow" else dk.cpu()
        hd_v = hs_v if cfg.kind == "cow" else dv.cpu()
        mh = m.cpu()
        reps, t_start = 0, time.perf_counter()
        while True:
            oracle.copy_blocks(hd_k, hs_k, mh, inplace=True)
            oracle.copy_blocks(hd_v, hs_v, mh, inplace=True)
            reps += 1
            el = time.perf_counter() - t_start
            if el >= args.cpu_seconds or reps >= 1000:
                break
        result["cpu_baseline"] = {
            "value": round(moved * reps / el / 1e9, 3),
            "unit": "GB/s",
            "cores": 1,
            "kind": "oracle",
            "sample": f"{reps} full {cfg.name} copies on host copies of the pools, {el:.1f} s wall, one thread",
        }
    return result


if __name__ == "__main__":
    main()

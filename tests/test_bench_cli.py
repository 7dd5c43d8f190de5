"""bench.py's command-line contract where no GPU is needed: more than one GPU
is refused with a message, a missing GPU is an error, and every workload name
the benchmark accepts resolves to a seeded layout."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.skipif(__import__("torch").cuda.is_available(), reason="checks the no-GPU error")
def test_no_gpu_is_an_error():
    r = _run("--steps", "1", "--warmup", "0")
    assert r.returncode != 0
    assert "GPU" in r.stderr


def test_every_workload_has_a_seeded_layout():
    sys.path.insert(0, ROOT)
    from pa_workloads import CONFIGS, make_layout
    from pa_workloads.layers import LAYER_CONFIGS
    from pa_workloads.prefill import PREFILL_CONFIGS, make_prefill_layout

    for name, cfg in CONFIGS.items():
        lay = make_layout(cfg)
        assert lay.context_lens.shape == (cfg.num_seqs,) and (lay.context_lens >= 1).all(), name
        assert (lay.block_tables >= 0).all() and (lay.block_tables < cfg.num_blocks).all(), name
    for name, p in PREFILL_CONFIGS.items():
        pl = make_prefill_layout(p)
        assert int(pl.query_start_loc[-1]) > 0, name
    for name, l in LAYER_CONFIGS.items():
        assert l.num_layers > 1 and l.base.name in CONFIGS, name

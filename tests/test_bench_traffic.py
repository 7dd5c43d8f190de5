"""The HBM traffic bench.py reports next to the roofline comes from the
committed counter summary (profiles/traffic.json): per launch, FETCH_SIZE and
WRITE_SIZE in KiB per dispatch, each scaled by the factor a plain device copy
of known size measured in the same run.  Checked here without a GPU: every
record's bytes follow from its counters by that rule, a record is only
reported while the kernel sources hash to the ones it was taken on, and a
workload without a record reports none."""

import json
import os

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _records():
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        return json.load(f)


def test_records_follow_the_counter_rule():
    recs = _records()
    assert recs, "no traffic records"
    for name, r in recs.items():
        assert r["kernel"] in bench.KERNEL_SOURCES, name
        want = (r["fetch_kib_per_dispatch"] * r["fetch_factor"] + r["write_kib_per_dispatch"] * r["write_factor"]) * 1024
        assert r["bytes_per_launch"] == pytest.approx(want, rel=1e-3), name
        # the calibration copy moves each byte once; on this part FETCH_SIZE
        # reads about half of what it moves and WRITE_SIZE all of it
        assert 0.9 <= r["write_factor"] <= 1.1 and 1.8 <= r["fetch_factor"] <= 2.2, name
        # measured traffic is never below the algorithmic bytes by more than rounding
        assert r["bytes_per_launch"] >= 0.99 * r["algorithmic_bytes_per_launch"], name


def test_reported_only_while_sources_match(monkeypatch):
    recs = _records()
    name, r = next(iter(recs.items()))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda kind="decode": r["source_hash"])
    assert bench.measured_traffic(name, r["kernel"]) == r["bytes_per_launch"]
    monkeypatch.setattr(bench, "kernel_source_hash", lambda kind="decode": "0" * 16)
    assert bench.measured_traffic(name, r["kernel"]) is None


def test_no_record_no_traffic():
    assert bench.measured_traffic("no_such_workload") is None

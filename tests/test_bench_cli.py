"""The bench's host-side contract (no GPU needed): it refuses more than one
GPU with a message and MTP-3 runs past its 32 iterations, reports profiled
traffic only for the kernel sources the profile was taken on, prices Stage
One's algorithmic bytes by the unit costs it documents, and measures
adjacent-step reuse by the page's definition."""
from __future__ import annotations

import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_profiled_traffic_follows_the_kernel_sources(tmp_path, monkeypatch):
    # The committed summary matches the committed sources.
    assert bench.profiled_traffic("gather_kernel", "matching") is not None
    assert bench.profiled_traffic("gather_kernel", "no-such-workload") is None
    # Any change to the gather's sources makes the figure stale.
    for f in bench.KERNEL_SOURCES["gather_kernel"]:
        data = open(os.path.join(bench.CSRC, f), "rb").read()
        (tmp_path / f).write_bytes(data + (b"\n// changed\n" if f.endswith(".hip") else b""))
    monkeypatch.setattr(bench, "CSRC", str(tmp_path))
    assert bench.profiled_traffic("gather_kernel", "matching") is None


def test_probe_sweep_counters_cover_every_batch_size():
    """The committed sweep summary holds counter bytes for each batch size the
    sweep runs, growing with the batch, and its B = 256 figure agrees with
    the separate B = 256 run."""
    per_b = [bench.profiled_traffic("stage1_kernel", "probe-sweep",
                                    f"traffic_bytes_per_launch_B{B}")
             for B in (32, 128, 256, 512, 1024)]
    assert all(v is not None for v in per_b)
    assert per_b == sorted(per_b)
    single = bench.profiled_traffic("stage1_kernel", "probe-sweep")
    assert abs(per_b[2] - single) <= 1e-3 * single
    assert bench.profiled_traffic("stage1_kernel", "probe-sweep",
                                  "traffic_bytes_per_launch_B7") is None


def test_mtp3_runs_past_its_iterations_are_refused():
    """MTP-3 is defined as 32 iterations from an empty buffer; the bench
    refuses warm-up + timed steps beyond that instead of replaying."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "mtp3",
                        "--warmup", "5", "--steps", "28"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2 and "32 iterations" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("B,S,Nq,lookups,visits,misses", [(1, 16, 1, 0, 0, 0),
                                                          (8, 2048, 1, 16384, 40000, 11000),
                                                          (3, 64, 4, 30, 70, 9)])
def test_stage_one_algorithmic_bytes(B, S, Nq, lookups, visits, misses):
    expect = (B * 2 * S * 4          # lifetimes read and written once per request
              + lookups * (4 + 4 + 1)  # id in, slot out, mask out
              + visits * 8           # bucket word and cached id per visit
              + misses * (12 + 8)    # install (C, F, Q) and miss-list entry
              + B * Nq * 4)          # miss count per token
    assert bench.stage1_algorithmic_bytes(B, S, Nq, lookups, visits, misses) == expect


def test_step_counts_are_validated():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "0"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "--steps" in r.stderr


def test_adjacent_step_reuse_follows_the_rate_definition():
    """The bench's adjacent-step reuse is the mean, over requests and steps,
    of the page's definition as the oracle's rate module states it."""
    from oracle import rates
    from workloads import make
    for name in ("tiny", "matching"):
        w = make(name, steps=6)
        expect = np.mean([rates.adjacent_reuse(w.topk[t - 1, b], w.topk[t, b])
                          for t in range(2, 6) for b in range(w.B)])
        assert bench.adjacent_step_reuse(w.topk, 2, 6) == pytest.approx(expect, abs=1e-12)
    assert bench.adjacent_step_reuse(w.topk, 0, 6) is None

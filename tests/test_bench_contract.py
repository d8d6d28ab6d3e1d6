"""Host-side checks of bench.py's contract (no GPU needed).

The single-GPU guard, the algorithmic byte counts behind the roofline (the
per-unit figures the design states: 132,868 B per (row, head) of decode at
d = 128, 1,796 B per (token, head) of verify input and output plus 1,028 B of
replay copy), the rule that measured HBM traffic is reported only for the
kernel sources and launch shape it was counted on, and the oracle baseline
leg on a tiny workload.
"""

import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_decode_bytes_per_unit():
    per_head = 2 * 128 * 128 * 4 + 3 * 128 * 2 + 128 * 4 + 4 + 128 * 4   # state in+out, q k v, alpha, beta, out
    assert per_head == 132868
    assert bench.decode_bytes(1, 1, 128, 128) == per_head + 4              # + the row's slot id
    assert bench.decode_bytes(64, 32, 128, 128) == 272113920               # the headline's bytes per launch


def test_verify_and_commit_bytes():
    state = 16 * 32 * 128 * 128 * 4
    per_tok = (2 * 128 + 128) * 2 + 128 * 4 + 4 + 128 * 4
    assert per_tok == 1796
    replay = 128 * 2 + 128 * 2 + 128 * 4 + 4
    assert replay == 1028
    meta = 16 * 4 + 17 * 4
    n_tok = 128
    assert bench.verify_bytes(n_tok, 16, 32, 128, 128, 0, 8) == state + n_tok * 32 * (per_tok + replay) + meta
    assert bench.verify_bytes(n_tok, 16, 32, 128, 128, 1, 8) == (state + n_tok * 32 * per_tok + meta
                                                                   + n_tok * 32 * 128 * 128 * 4)
    acc = np.array([3, 0, 8, 1], np.int32)
    live = 3 * 32 * 128 * 128 * 4
    assert bench.commit_bytes(acc, 32, 128, 128, 0) == 2 * live + 12 * 32 * replay + 4 * 8
    assert bench.commit_bytes(acc, 32, 128, 128, 1) == 2 * live + 4 * 8


def _counter_fields():
    fields = {}
    for line in open(bench.COUNTERS_FILE):
        if ":" in line and not line.startswith("#"):
            key, val = line.split(":", 1)
            fields[key.strip()] = val.strip()
    return fields


def test_traffic_only_for_the_counted_source_and_shape(monkeypatch):
    f = _counter_fields()
    tile = tuple(int(x.split()[1]) for x in f["launch"].split(","))
    monkeypatch.setattr(bench, "kernel_source_sha256", lambda: f["kernel_source_sha256"])
    assert bench.stored_traffic(tile) == int(f["hbm_bytes_per_launch"])
    assert bench.stored_traffic((tile[0] * 2, tile[1])) is None
    monkeypatch.setattr(bench, "kernel_source_sha256", lambda: "0" * 64)
    assert bench.stored_traffic(tile) is None
    # the counted traffic is within a fraction of a percent of the algorithmic bytes
    assert abs(int(f["hbm_bytes_per_launch"]) / bench.decode_bytes(64, 32, 128, 128) - 1) < 0.01


def test_cpu_baseline_leg_runs_the_oracle():
    w = synth.make(1, 4, 64, 64, num_slots=4, state_std=0.02, seed=3, name="tiny")
    r = bench.cpu_baseline(w, seconds_scale=0.01)
    assert r["kind"] == "oracle" and r["unit"] == "steps/s"
    assert r["cores"] == len(os.sched_getaffinity(0)) and r["value"] > 0
    assert r["cpu_count"] == os.cpu_count() and r["cpu_model"]
    assert r["one_core_steps_per_s"] > 0 and r["b1_us_per_step_all_cores"] > 0 and r["b1_us_per_step_one_core"] > 0
    for part in r["detail"].values():
        assert len(part["samples_steps_per_s"]) == 3
        assert part["steps_per_s"] == round(sorted(part["samples_steps_per_s"])[1], 3)
    assert "steps" in r["sample"] and "median of 3" in r["sample"]

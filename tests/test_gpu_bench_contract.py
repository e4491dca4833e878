"""bench.py's JSON line for every workload it times, run in this process with
a few steps: the fields a reader of the line relies on are present and
consistent (value from the timed steps, the roofline fraction from its own
figures, the parity figure within the path's bound).
"""
import argparse
import json

import pytest
import torch

import bench
import synth
from gpu_common import dev, say

pytestmark = pytest.mark.gpu


def _args(workload):
    return argparse.Namespace(gpus=1, steps=3, warmup=1, workload=workload, no_cpu_baseline=True,
                              copy_calibration=0, segmented=False, prefill_only=True)


def _common(rec, workload):
    json.dumps(rec)   # serialisable as one line
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline"):
        assert key in rec, key
    assert rec["n_gpus"] == 1 and rec["steps"] == 3 and rec["warmup"] == 1
    assert rec["vs_baseline"] is None and rec["data"] == "synthetic"
    assert rec["config"]["workload"] == workload
    r = rec["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic", "copy_GBs", "frac_of_copy", "spread"):
        assert key in r, key
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == bench.HBM_PEAK_GBS
    assert r["achieved"] > 0 and r["frac"] == pytest.approx(r["achieved"] / r["peak"])
    assert r["frac_of_copy"] == pytest.approx(r["achieved"] / r["copy_GBs"])
    assert 0 < r["frac"] < 1 and 0 < r["copy_GBs"] < r["peak"]
    s = r["spread"]
    assert s["replays"] == 11 and s["p10_us"] <= s["median_us"] <= s["p90_us"] and s["first_replay_us"] > 0
    assert r["kernel_ms"] == pytest.approx(s["median_us"] / 1e3)
    assert "cpu_baseline" not in rec


def test_prefill_line():
    say("bench contract: prefill_t4576_h0")
    w = synth.WORKLOADS["prefill_t4576_h0"]
    dev()
    rec = bench.with_copy_yardstick(bench.bench_prefill(w, _args(w.name), torch), torch)
    _common(rec, w.name)
    assert rec["value"] == pytest.approx(w.B * w.T / (rec["ms_per_step"] * 1e-3))
    assert rec["route"].startswith("gdn_wy_prep_kernel+gdn_spine_kernel")
    assert rec["parity_max_rel_err_sampled_heads"] <= 2e-2


def test_segmented_prefill_line():
    say("bench contract: prefill_t4576_hv6 --segmented")
    w = synth.WORKLOADS["prefill_t4576_hv6"]
    args = _args(w.name)
    args.segmented = True
    rec = bench.with_copy_yardstick(bench.bench_prefill(w, args, torch), torch)
    _common(rec, w.name)
    assert rec["config"]["entry"] == "gdn_chunk_prefill_segmented"
    assert "gdn_segment_combine_kernel" in rec["route"], rec["route"]
    assert rec["parity_max_rel_err_sampled_heads"] <= 2e-2


def test_verify_line():
    say("bench contract: verify_k4_b16")
    w = synth.WORKLOADS["verify_k4_b16"]
    rec = bench.with_copy_yardstick(bench.bench_verify(w, _args(w.name), torch), torch)
    _common(rec, w.name)
    assert rec["value"] == pytest.approx(rec["roofline"]["achieved"])
    assert rec["parity_max_rel_err_out"] <= 2e-2
    assert rec["fold"]["kernel_ms"] > 0 and rec["fold"]["spread"]["replays"] == 11


def test_step_line():
    say("bench contract: step_b16")
    w = synth.WORKLOADS["step_b16"]
    rec = bench.with_copy_yardstick(bench.bench_step(w, _args(w.name), torch), torch)
    _common(rec, w.name)
    assert rec["parity_max_rel_err_out"] <= 2e-2 and rec["parity_max_rel_err_state"] <= 1e-4


def test_ba_line():
    say("bench contract: ba_gates_t4576")
    name = synth.BA_WORKLOAD["name"]
    rec = bench.with_copy_yardstick(bench.bench_ba(_args(name), torch), torch)
    _common(rec, name)
    assert rec["parity_max_rel_err_sampled_tokens"] <= 1e-4


def test_default_line_carries_verify_and_fold():
    """The default run (what the driver times) prints one JSON line whose extra
    keys hold the K = 4 verify's and the fold's HBM rooflines and the 6-v-head
    layer share through the plain spine and the segment scan."""
    import os
    import subprocess
    import sys
    say("bench contract: default line (subprocess)")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "bench.py", "--steps", "3", "--warmup", "1", "--no-cpu-baseline"],
                       cwd=root, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1
    rec = json.loads(lines[0])
    assert rec["config"]["workload"] == "prefill_t4576_h0"
    for key in ("decode_verify_k4", "fold_k4"):
        rf = rec[key]["roofline"]
        assert rf["bound"] == "hbm" and rf["unit"] == "GB/s"
        assert 0 < rf["frac"] < 1 and rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"])
    assert rec["decode_verify_k4"]["parity_max_rel_err_out"] <= 2e-2
    nar = rec["prefill_hv6"]
    assert nar["config"]["Hv"] == 6 and nar["config"]["Hk"] == 2
    assert "gdn_segment_combine_kernel" in nar["segment_scan"]["route"]
    assert "segment" not in nar["plain_spine"]["route"].split(" ")[0]
    assert nar["speedup"] == pytest.approx(nar["plain_spine"]["ms_per_call"] / nar["segment_scan"]["ms_per_call"])
    for k in ("plain_spine", "segment_scan"):
        assert nar[k]["parity_max_rel_err_sampled_heads"] <= 2e-2

"""The benchmark's report: one JSON line with the fields its readers rely on, from a short
run on a small layer (N=1024, H=2, d=64) in a child process."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_prints_one_json_line_with_roofline_and_cpu_baseline():
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny_sparse",
           "--steps", "3", "--warmup", "1", "--dense-steps", "1", "--cold-steps", "1",
           "--cpu-budget", "1", "--cpu-single-budget", "0.5"]
    print("bench:", " ".join(cmd[1:]), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout[-3000:]
    rep = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline", "stage_ms"):
        assert key in rep, key
    assert rep["n_gpus"] == 1 and rep["steps"] == 3 and rep["warmup"] == 1
    assert rep["unit"] == "ms/layer" and rep["higher_is_better"] is False
    assert rep["value"] == rep["ms_per_step"] and rep["value"] > 0
    assert rep["config"]["workload"] == "tiny_sparse"
    # every stage of the step was timed, the two on the second stream included
    for st in ("mask_pool", "mask_select", "fwd", "bwd_dq", "bwd_dkdv", "fwd_prep_overlapped",
               "bwd_prep_overlapped"):
        assert rep["stage_ms"][st] > 0, st
    rf = rep["roofline"]
    assert rf["bound"] in ("hbm", "mfma") and rf["unit"] in ("GB/s", "TFLOP/s")
    assert rf["peak"] in (8000.0, 2500.0)
    assert rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"])
    assert 0 < rf["frac"] < 1
    cb = rep["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] >= 1 and cb["value"] > 0
    assert cb["unit"] == rep["unit"] and cb["sample"]
    assert cb["host_logical_cpus"] >= 1 and cb["usable_cpus"] >= 1
    assert cb["single_thread_one_head_ms"] > 0 and cb["single_thread_sample"]
    # the mask's headline rate is the cold-cache one; the warm figure is labelled apart
    assert rep["mask_ms"] > 0 and rep["mask_ms_warm"] > 0
    assert 0 < rep["mask_hbm_frac"] < 1 and 0 < rep["mask_hbm_frac_warm_cache"]
    assert "fp16" in rep["config"]["precision"]

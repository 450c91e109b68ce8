"""bench.py end to end on one small workload: it runs, and its last line keeps the one-line JSON
contract (metric, value, roofline with the HBM bound, the CPU baseline field, the references)."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
pytestmark = pytest.mark.gpu


def test_bench_prints_the_contract_line():
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "llama_layer_n8_rank0",
           "--steps", "3", "--warmup", "1", "--no-cpu-baseline", "--no-extra-workloads"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-3000:]
    rec = json.loads(r.stdout.strip().splitlines()[-1])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline", "ceiling", "mix_reference"):
        assert key in rec, key
    assert rec["n_gpus"] == 1 and rec["steps"] == 3 and rec["warmup"] == 1
    assert rec["unit"] == "params/s" and rec["value"] > 0 and rec["higher_is_better"] is True
    assert rec["config"]["workload"] == "llama_layer_n8_rank0"
    roof = rec["roofline"]
    assert roof["bound"] == "hbm" and roof["peak"] == 8000.0 and roof["unit"] == "GB/s"
    assert 0.0 < roof["frac"] < 1.0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    for k in ("read", "write", "copy", "read2_write1"):
        assert rec["ceiling"][k]["GBps"] > 0
    assert rec["mix_reference"]["flushed"] is True        # a small slice runs with the flush


def test_fp32_gradient_paths_carry_their_replica():
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "llama_layer_n8_rank0",
           "--path", "accumulate", "--steps", "2", "--warmup", "1", "--no-cpu-baseline",
           "--no-ceiling"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-3000:]
    rec = json.loads(r.stdout.strip().splitlines()[-1])
    calls = [st["call"] for st in rec["config"]["stages"]]
    assert calls[-1].startswith("adamw_shard_step_f32grad_blocked")
    ref = rec["mix_reference"]
    assert ref["flushed"] == ("flush" in rec["config"]["timing"])   # flushed as the stages are
    assert ref["f32grad_step_bytes"]["GBps"] > 0 and ref["f32grad_step_bytes"]["ms"] > 0

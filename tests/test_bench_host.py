"""Host-side checks of bench.py that need no GPU: the one-GPU contract and the counter digest."""

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    for n in (2, 8):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                           capture_output=True, text=True, timeout=120)
        assert r.returncode == 2
        assert "one GPU" in r.stderr and r.stdout == ""


def test_source_digest_ignores_comments_only(tmp_path):
    a = tmp_path / "a.hip"
    b = tmp_path / "b.hip"
    c = tmp_path / "c.hip"
    a.write_text("// note\nint f(int x) { return x + 1; } /* block\n comment */\n")
    b.write_text("// another note\n\nint f(int x)  {\n  return x + 1;\n}\n")
    c.write_text("int f(int x) { return x + 2; }\n")
    assert bench.source_digest(str(a)) == bench.source_digest(str(b))
    assert bench.source_digest(str(a)) != bench.source_digest(str(c))


def test_counter_traffic_is_reported_only_for_the_measured_code(tmp_path, monkeypatch):
    # A traffic entry counts only while its digest matches the kernel code; otherwise the bench
    # reports no traffic (the counters must be taken again).
    src = tmp_path / "k.hip"
    src.write_text("int f() { return 1; }\n")
    table = tmp_path / "traffic.json"
    table.write_text(json.dumps({"w": {"bytes_per_launch": 123,
                                       "kernel_source_sha256_16": bench.source_digest(str(src))}}))
    monkeypatch.setattr(bench, "PROFILE_TRAFFIC", str(table))
    assert bench.counter_traffic("w", str(src)) == 123
    assert bench.counter_traffic("other", str(src)) is None
    src.write_text("int f() { return 2; }\n")
    assert bench.counter_traffic("w", str(src)) is None


def test_host_cores_are_stated():
    c = bench.host_cores()
    assert c["os_cpu_count"] >= 1 and c["affinity"] >= 1
    assert 1 <= c["usable"] <= c["affinity"]
    if c["cgroup_quota"] is not None:
        assert c["usable"] <= c["cgroup_quota"]


def test_cpu_baseline_legs_report_the_contract_fields():
    # Tiny samples: the legs' structure, not their speed.
    one = bench.cpu_baseline_single("p1000003_n8_rank3", seconds=0.2, sample=4096)
    assert one["kind"] == "oracle" and one["cores"] == 1 and one["unit"] == "params/s"
    assert one["value"] > 0 and "4096 elements" in one["sample"]
    par = bench.cpu_baseline("p1000003_n8_rank3", 2, seconds=0.2, chunk=8192)
    assert par["kind"] == "oracle" and par["cores"] == 2 and par["value"] > 0
    assert set(par["host"]) == {"os_cpu_count", "affinity", "cgroup_quota", "usable"}
    assert "2 processes" in par["sample"]


def test_failed_child_measurement_is_recorded_not_fatal():
    # A measurement that runs in a child process and fails (an unknown layout; without a GPU the
    # child stops even earlier, also with status 1) comes back as an error record, so the bench
    # still prints its line with the headline.
    import argparse
    args = argparse.Namespace(workload="p1000003_n8_rank3", steps=1, warmup=0, evict_mb=-1,
                              no_copy_reference=True)
    rec = bench.run_child(args, "workload:p1000003_n8_rank3:no_such_layout")
    assert rec == {"error": "exit status 1"}


def test_layout_keys():
    assert bench.traffic_key("w") == "w"
    assert bench.traffic_key("w", "separate") == "w:separate"
    assert bench.traffic_key("w", "interleaved") == "w:interleaved"
    assert set(bench.LAYOUT_DESCRIPTION) == {"blocked", "separate", "interleaved"}
    assert all(lay in bench.LAYOUT_DESCRIPTION for _, lay in bench.EXTRA_WORKLOADS)

"""Host-side logic of bench.py: the one-GPU guard and the traffic record (no GPU)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _record(sha, nbytes=123456):
    return {bench.DOMINANT: {"kernel": "w4a16_dot2_kernel", "kernel_source_sha": sha,
                             "fetch_kib_per_dispatch": 1.0, "write_kib_per_dispatch": 1.0,
                             "fetch_factor": 2.0, "write_factor": 1.0, "bytes_per_launch": nbytes}}


def test_traffic_needs_a_record_of_the_current_sources(tmp_path):
    p = tmp_path / "traffic.json"
    assert bench.measured_traffic(str(p)) is None  # no record
    p.write_text(json.dumps(_record(bench._kernel_source_sha())))
    assert bench.measured_traffic(str(p)) == 123456
    p.write_text(json.dumps(_record("0" * 16)))
    assert bench.measured_traffic(str(p)) is None  # counters taken on other sources
    p.write_text(json.dumps({"other_workload": _record(bench._kernel_source_sha())[bench.DOMINANT]}))
    assert bench.measured_traffic(str(p)) is None


def test_committed_traffic_record_is_consistent():
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        t = json.load(f)[bench.DOMINANT]
    assert t["kernel"] == "w4a16_dot2_kernel"
    # bytes = (FETCH_SIZE x fetch factor + WRITE_SIZE x write factor) KiB, from
    # the unrounded figures: the record rounds the KiB to 0.1 and the factors to
    # 0.001 (or finer)
    est = (t["fetch_kib_per_dispatch"] * t["fetch_factor"] + t["write_kib_per_dispatch"] * t["write_factor"]) * 1024
    slack = (0.05 * (t["fetch_factor"] + t["write_factor"])
             + 0.0005 * (t["fetch_kib_per_dispatch"] + t["write_kib_per_dispatch"])) * 1024
    assert abs(t["bytes_per_launch"] - est) <= slack
    # measured traffic of a streaming kernel cannot be below its algorithmic bytes
    N, K, G = 6144, 5120, 128
    algo = N * K // 2 + (K // G) * N * 2 + K * 2 + N * 2
    assert algo == 16242688
    assert t["bytes_per_launch"] >= algo

"""bench.py's host-side contract that needs no GPU: one GPU only, and the
counter-measured traffic is tied to the GEMM source it was taken on."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line for a run that did not happen


def test_measured_traffic_follows_the_gemm_source(monkeypatch):
    sys.path.insert(0, ROOT)
    import bench

    name = next(iter(bench.MEASURED_TRAFFIC))
    m = bench.MEASURED_TRAFFIC[name]
    expect = int(round((m["fetch_kib"] * bench.FETCH_SCALE + m["write_kib"] * bench.WRITE_SCALE) * 1024))
    if m["gemm_sha256"] == bench.gemm_source_sha():
        assert bench.measured_traffic(name) == expect
    # any other GEMM source: the figure no longer applies
    monkeypatch.setattr(bench, "gemm_source_sha", lambda: "0" * 128)
    assert bench.measured_traffic(name) is None
    assert bench.measured_traffic("no_such_workload") is None
    json.dumps(bench.MEASURED_TRAFFIC)  # plain data

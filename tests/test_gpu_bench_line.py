"""bench.py end to end on a small workload: one JSON line with the keys and
types its readers rely on (the throughput, the roofline of the dominant
stage, the route, dispatch and combine stages against HBM, the CPU oracle
baseline)."""
import json
import os
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_json_line(monkeypatch, capsys):
    print("bench.py on tiny_e8k2_f32", flush=True)
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import bench  # run in this process: no child program is started

    monkeypatch.setattr(sys, "argv", ["bench.py", "--steps", "3", "--warmup", "2",
                                      "--workload", "tiny_e8k2_f32", "--no-dense",
                                      "--no-decode", "--cpu-sample", "64"])
    capsys.readouterr()
    bench.main()
    out = capsys.readouterr().out
    lines = [l for l in out.splitlines() if l.strip().startswith("{")]
    assert len(lines) == 1, out
    j = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline", "route_roofline", "combine_roofline", "stage_us"):
        assert key in j, key
    assert j["n_gpus"] == 1 and j["steps"] == 3 and j["warmup"] == 2
    assert j["unit"] == "tokens/s" and j["higher_is_better"] is True and j["dtype"] == "f32"
    assert j["config"]["workload"] == "tiny_e8k2_f32" and j["config"]["tokens"] == 64
    assert j["value"] > 0 and j["ms_per_step"] > 0
    assert abs(j["value"] - 64 / (j["ms_per_step"] * 1e-3)) <= 1e-3 * j["value"]
    st = j["step_ms"]
    assert 0 < st["min"] <= st["median"] and st["median"] == j["ms_per_step"]
    assert j["scrubbed"]["median_ms"] > 0 and j["scrubbed"]["min_ms"] <= j["scrubbed"]["median_ms"]
    roof = j["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in roof, key
    assert roof["bound"] in ("hbm", "mfma", "alu")
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    for stage in ("route_roofline", "combine_roofline"):
        s = j[stage]
        assert s["bound"] == "hbm" and s["unit"] == "GB/s" and s["achieved"] > 0
    d = j["dispatch_roofline"]  # a few KB at this size: flagged as latency-bound
    assert d["bound"] == "latency" and d["unit"] == "GB/s" and d["achieved"] > 0
    assert d["algorithmic_bytes"] == 64 * 2 * 8 + 2 * 8 * 4 + 9 * 4 + 64 * 2 * 4 + 8
    cpu = j["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1 and cpu["sample"]
    assert cpu["host_cores"] == len(os.sched_getaffinity(0)) and cpu["cpu_model"]
    assert set(j["stage_us"]) == {"route", "dispatch", "expert_ffn", "combine"}


def test_decode_roofline_object():
    """The decode-shape layer's HBM figure that the bench line carries: whole
    layer, touched experts' weights only generated."""
    print("bench.decode_roofline", flush=True)
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import bench

    d = bench.decode_roofline(steps=2, warmup=1)
    assert d["bound"] == "hbm" and d["unit"] == "GB/s" and d["peak"] == bench.PEAK_HBM_GBS
    assert abs(d["frac"] - d["achieved"] / d["peak"]) < 1e-3
    assert 0 < d["ms_min"] <= d["ms_median"]
    assert 100 <= d["experts_touched"] <= 256
    assert d["algorithmic_bytes"] > d["experts_touched"] * 3 * 7168 * 2048 * 2

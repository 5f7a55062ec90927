"""The benchmark's one JSON line, produced on the GPU for the tiny decoder.

Runs bench.main() in this process (no second process on the GPU) with a short
decode and a small CPU-baseline budget, and checks the line's fields: the
metric and its unit, the whole-job throughput, the roofline block whose
fraction is achieved / peak with the algorithmic bytes of the timed launch,
and the CPU-oracle baseline.
"""
import json
import sys

import pytest

import bench
from persistent_decode_monokernel_amd import synth

pytestmark = pytest.mark.gpu

STEPS = 8


def test_bench_json_line(capsys, monkeypatch):
    monkeypatch.setattr(sys, "argv", ["bench.py", "--workload", "tiny", "--steps", str(STEPS), "--warmup", "2",
                                      "--cpu-budget", "1"])
    bench.main()
    lines = [l for l in capsys.readouterr().out.splitlines() if l.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
                "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["metric"] == bench.METRIC and d["unit"] == "tokens/s"
    assert d["n_gpus"] == 1 and d["steps"] == STEPS and d["warmup"] == 2 and d["status"] == 0
    assert d["value"] > 0 and d["higher_is_better"] is True and d["dtype"] == "f16" and d["data"] == "synthetic"
    assert d["config"]["workload"].startswith("tiny") and "model" not in d["config"]
    assert abs(d["ms_per_step"] * d["value"] - 1e3) < 1e-6 * 1e3

    r = d["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    s = synth.WORKLOADS["tiny"].shape
    nbytes = bench.bytes_per_launch(s, synth.WORKLOADS["tiny"].n_prompt, STEPS)
    assert d["kernel"]["algorithmic_bytes_per_launch"] == nbytes
    assert abs(r["achieved"] - nbytes / (d["kernel"]["launch_ms"] / 1e3) / 1e9) < 1e-6 * r["achieved"]
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-12
    assert r["traffic"] is None  # counters are stored for the ~2B workload only

    c = d["cpu_baseline"]
    assert c is not None and c["kind"] == "oracle" and c["value"] > 0 and c["cores"] >= 1
    assert "C++" in c["implementation"] and c["nproc"] >= c["cores"] and c["cpu_model"]
    assert c["unit"] == "tokens/s" and c["sample"]

"""bench.py's output contract on a short run: one JSON line on stdout with
the keys and types the benchmark line promises, the headline stage's
roofline (achieved / peak = frac, HBM traffic from the committed counters
when the sources match), and the oracle's CPU baseline."""
import json
import os
import subprocess
import sys

import pytest

from gpu_util import say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_json_line():
    say("bench.py --steps 3 --warmup 1 --stages softmax_f32,attn_nc --cpu-seconds 2")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "1",
                        "--min-warmup-s", "0", "--stages", "softmax_f32,attn_nc", "--no-box-references",
                        "--cpu-seconds", "2"], capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout  # exactly one line: the result
    d = json.loads(lines[0])
    for key, typ in [("metric", str), ("value", float), ("unit", str), ("n_gpus", int), ("steps", int),
                     ("warmup", int), ("ms_per_step", float), ("higher_is_better", bool), ("scaling", str),
                     ("dtype", str), ("data", str), ("config", dict), ("roofline", dict), ("cpu_baseline", dict)]:
        assert isinstance(d[key], typ), (key, d[key])
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["higher_is_better"] is True and d["vs_baseline"] is None and d["data"] == "synthetic"
    assert d["unit"] == "GB/s" and d["dtype"] == "f32"
    assert "workload" in d["config"] and "model" not in d["config"]
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert rf["achieved"] == d["value"]
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert 0.3 < rf["frac"] < 1.0, rf  # an HBM-bound kernel on this chip
    if rf["traffic"] is not None:  # counters taken with these sources
        assert abs(rf["traffic"] / rf["algorithmic_units_per_launch"] - 1.0) < 0.02
    nc = d["paths"]["attn_nc"]["roofline"]
    assert nc["bound"] == "mfma" and nc["unit"] == "TFLOP/s" and 0.2 < nc["frac"] < 1.0, nc
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["unit"] == "GB/s" and cb["cores"] >= 1 and cb["value"] > 0
    assert isinstance(cb["sample"], str) and cb["sample"]
    assert "cpu_model" in cb

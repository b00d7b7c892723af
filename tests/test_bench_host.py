"""bench.py's host-side logic on the CPU: the one-GPU refusal, turning two
rocprofv3 counter files into HBM bytes per launch (each counter scaled by
what it reads for a plain 1 GiB copy), and reporting those bytes only while
the kernel sources are the ones the counters were taken with."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line for a run that did not happen


def _csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Grid_Size", "Counter_Value"])
        w.writeheader()
        for name, grid, v in rows:
            w.writerow({"Kernel_Name": name, "Grid_Size": grid, "Counter_Value": v})


def test_ingest_counters_scales_by_the_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    copy = "__amd_rocclr_copyBuffer"
    sm = "void tea::row_softmax_kernel<false, 256, 32, true, 8, 256, 0>(...)"
    causal = "void tea::attn_fwd_kernel<128, 64, 8, true>(...)"
    # the copy of 1 GiB reads 2^19 KiB on the FETCH counter (a factor 2 to
    # calibrate away) and 2^20 KiB on WRITE; the softmax twice, the causal
    # attention at its own grid and at another grid (another stage)
    _csv(tmp_path / "fetch.csv", [(copy, 1 << 20, 524288.0), (sm, 65536 * 256, 1048576.0), (sm, 65536 * 256, 1048580.0),
                                 (causal, 2048 * 512, 300000.0), (causal, 32 * 512, 99.0)])
    _csv(tmp_path / "write.csv", [(copy, 1 << 20, 1048576.0), (sm, 65536 * 256, 2097152.0),
                                 (sm, 65536 * 256, 2097152.0), (causal, 2048 * 512, 131072.0), (causal, 32 * 512, 7.0)])
    out = bench.ingest_counters(str(tmp_path / "fetch.csv"), str(tmp_path / "write.csv"), "cmd")
    assert out["_calibration"]["read_factor"] == pytest.approx(2.0)
    assert out["_calibration"]["write_factor"] == pytest.approx(1.0)
    s = out["softmax_f32"]
    assert s["read_bytes"] == int(1048578.0 * 1024 * 2.0)  # mean of the two dispatches, scaled
    assert s["write_bytes"] == 2097152 * 1024
    assert s["bytes_per_launch"] == s["read_bytes"] + s["write_bytes"]
    c = out["attn_causal"]
    assert c["read_bytes"] == int(300000.0 * 1024 * 2.0)  # only the dispatches at the causal grid
    assert c["source_hash"] == bench.source_hash("attn_fwd")
    assert "decode" not in out  # stages without counters are left out, not zero
    assert json.load(open(tmp_path / "traffic.json")) == out


def test_measured_traffic_follows_the_source_hash(tmp_path, monkeypatch):
    f = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    live = bench.source_hash("row_softmax")
    f.write_text(json.dumps({"softmax_f32": {"source_hash": live, "bytes_per_launch": 123},
                             "softmax_bf16": {"source_hash": "0" * 16, "bytes_per_launch": 456}}))
    assert bench.measured_traffic("row_softmax", "softmax_f32") == 123
    assert bench.measured_traffic("row_softmax", "softmax_bf16") is None  # taken with other sources
    assert bench.measured_traffic("row_softmax", "softmax_long_f32") is None  # never taken
    f.write_text("not json")
    assert bench.measured_traffic("row_softmax", "softmax_f32") is None


def test_every_stage_has_kernels_and_sources():
    for stage, parts in bench.STAGE_KERNELS.items():
        assert parts, stage
        assert bench.STAGE_SOURCE[stage] in bench.KERNEL_SOURCES, stage
    for kernel, files in bench.KERNEL_SOURCES.items():
        for p in files:
            assert os.path.exists(os.path.join(ROOT, p)), (kernel, p)

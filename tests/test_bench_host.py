"""Host-side logic of bench.py (no GPU): the single-GPU guard, the gate that
reports recorded HBM traffic only for the kernel sources it was measured on,
and the per-call statistics."""
import json
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_recorded_traffic_only_for_the_measured_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.recorded_traffic("nothing_recorded", "wkv_forward") is None
    body = "# HBM traffic\n\nsource-sha256: {}\ntraffic-bytes-per-call: wkv_forward=300 wkv_backward=500\n"
    (tmp_path / "hbm_traffic_same.md").write_text(body.format(bench.kernel_source_hash()))
    assert bench.recorded_traffic("same", "wkv_forward") == 300
    assert bench.recorded_traffic("same", "wkv_backward") == 500
    assert bench.recorded_traffic("same", "wkv_step") is None
    (tmp_path / "hbm_traffic_other.md").write_text(body.format("0" * 64))
    assert bench.recorded_traffic("other", "wkv_forward") is None


def test_source_hash_covers_the_kernels_and_the_header():
    h = bench.kernel_source_hash()
    assert len(h) == 64 and h == bench.kernel_source_hash()


def test_call_statistics_in_microseconds():
    st = bench.stats_us([0.1, 0.2, 0.3, 0.4])
    assert np.isclose(st["mean"], 250.0) and np.isclose(st["median"], 250.0)
    assert st["p10"] < st["median"] < st["p90"]

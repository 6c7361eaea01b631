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
    assert bench.recorded_traffic("nothing_recorded", "wkv_forward", "rwkv4") is None
    body = "# HBM traffic\n\nsource-sha256: {}\ntraffic-bytes-per-call: wkv_forward=300 wkv_backward=500\n"
    (tmp_path / "hbm_traffic_same.md").write_text(body.format(bench.kernel_source_hash("rwkv4")))
    assert bench.recorded_traffic("same", "wkv_forward", "rwkv4") == 300
    assert bench.recorded_traffic("same", "wkv_backward", "rwkv4") == 500
    assert bench.recorded_traffic("same", "wkv_step", "rwkv4") is None
    assert bench.recorded_traffic("same", "wkv_forward", "matrix") is None  # another family's sources
    (tmp_path / "hbm_traffic_other.md").write_text(body.format("0" * 64))
    assert bench.recorded_traffic("other", "wkv_forward", "rwkv4") is None


def test_source_hash_covers_each_familys_kernel_files(tmp_path, monkeypatch):
    """Each family hashes the files that define its kernels; a change to any of them changes it."""
    hashes = {f: bench.kernel_source_hash(f) for f in bench.KERNEL_FILES}
    assert all(len(h) == 64 for h in hashes.values()) and len(set(hashes.values())) == len(hashes)
    csrc = os.path.join(ROOT, "rwkv_wkv_mixing_amd", "csrc")
    for family, files in bench.KERNEL_FILES.items():
        for name in files:
            assert os.path.exists(os.path.join(csrc, name)), name
    fake = tmp_path / "rwkv_wkv_mixing_amd" / "csrc"
    fake.mkdir(parents=True)
    for name in os.listdir(csrc):
        (fake / name).write_bytes(open(os.path.join(csrc, name), "rb").read())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.kernel_source_hash("rwkv4") == hashes["rwkv4"]
    (fake / "wkv_bwd.hip").write_bytes(b"changed")
    assert bench.kernel_source_hash("rwkv4") != hashes["rwkv4"]
    assert bench.kernel_source_hash("matrix") == hashes["matrix"]


def test_call_statistics_in_microseconds():
    st = bench.stats_us([0.1, 0.2, 0.3, 0.4])
    assert np.isclose(st["mean"], 250.0) and np.isclose(st["median"], 250.0)
    assert st["p10"] < st["median"] < st["p90"]

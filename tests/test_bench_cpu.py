"""CPU checks of bench.py's host logic: the one-GPU contract, the FLOP
convention, and the lookup of committed HBM counter figures."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from io_aware_tiled_attn_amd import workloads as wl  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_flop_convention():
    w = wl.WORKLOADS["bf16_n4k_d128_causal"]
    fwd, bwd = bench.flops(w)
    assert fwd == 4.0 * 4 * 32 * 4096 * 4096 * 128 * 0.5
    assert bwd == 2.5 * fwd
    w2 = wl.WORKLOADS["bf16_n1k_d64"]
    assert bench.flops(w2)[0] == 4.0 * 8 * 16 * 1024 * 1024 * 64


def test_traffic_lookup(tmp_path, monkeypatch):
    sha = bench.kernel_source_hash()
    data = {"source_sha": sha, "kernels": {"k": {"w": {"bytes_per_launch": 123}}}}
    f = tmp_path / "t.json"
    f.write_text(json.dumps(data))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("k", "w") == 123
    assert bench.measured_traffic("k", "other") is None
    assert bench.measured_traffic("other", "w") is None
    data["source_sha"] = "0" * 16
    f.write_text(json.dumps(data))
    assert bench.measured_traffic("k", "w") is None      # stale once the kernels change
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.measured_traffic("k", "w") is None


def test_committed_traffic_file_is_well_formed():
    with open(bench.TRAFFIC_FILE) as f:
        data = json.load(f)
    assert len(data["source_sha"]) == 16 and data["copy_bytes"] > 0
    assert data["kernels"]["fa_fwd_bf16_kernel"]["bf16_n4k_d128_causal"]["bytes_per_launch"] > 0
    for entries in data["kernels"].values():
        for e in entries.values():
            assert e["bytes_per_launch"] == pytest.approx(e["read_bytes"] + e["write_bytes"], abs=2)

"""Host logic of bench.py (no GPU): the one-GPU contract and the stored traffic lookup."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_lookup_requires_the_measured_source(tmp_path, monkeypatch):
    good = bench._source_sha("gemm.h")
    entries = [{"workload": "d32", "stage": "down_dgrad", "source": "gemm.h", "source_sha": good,
                "hbm_bytes_per_launch": 123},
               {"workload": "d32", "stage": "up_fwd", "source": "gemm.h", "source_sha": "0" * 16,
                "hbm_bytes_per_launch": 456}]
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(entries))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("d32", "down_dgrad") == 123
    assert bench.measured_traffic("d32", "up_fwd") is None      # kernel changed since measured
    assert bench.measured_traffic("gpt2", "down_dgrad") is None  # other workload
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.measured_traffic("d32", "down_dgrad") is None


def test_stored_traffic_entries_name_existing_sources():
    entries = json.load(open(bench.TRAFFIC_FILE))
    assert entries
    for e in entries:
        assert os.path.exists(os.path.join(bench.CSRC, e["source"]))
        assert e["hbm_bytes_per_launch"] > 0
        assert e["stage"] in bench.TRAFFIC_KERNELS

"""bench.py's contract on the CPU: the one-GPU refusal for --gpus N > 1, a clear
failure without a GPU, and the traffic record used only for matching sources."""
from __future__ import annotations

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _bench("--gpus", "8")
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single MI355X" in r.stderr


def test_no_gpu_fails_loudly():
    import torch
    if torch.cuda.is_available():
        return
    r = _bench("--steps", "1", "--warmup", "0")
    assert r.returncode != 0
    assert "needs a GPU" in r.stderr


def test_traffic_record_needs_the_measured_sources(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    rec = {"source_hash": "not-these-sources",
           "workloads": {"w": {"hbm_bytes_per_launch": 123}}}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.recorded_traffic("w") is None
    rec["source_hash"] = bench.kernel_source_hash()
    f.write_text(json.dumps(rec))
    assert bench.recorded_traffic("w") == 123
    assert bench.recorded_traffic("other") is None

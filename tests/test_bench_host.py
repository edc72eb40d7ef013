"""CPU checks of bench.py's contract pieces that need no GPU: it refuses runs
on more than one GPU with a message, and it reports the rocprofv3 HBM traffic
only while the kernel sources and weight layout are the ones the counters
were taken on."""
import importlib.util
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_only_while_sources_and_layout_match(monkeypatch):
    B = _bench()
    rec = json.load(open(os.path.join(ROOT, "profiles", "gemm1_decode_traffic.json")))
    monkeypatch.setattr(B, "sources_sha256", lambda: rec["source_sha256"])
    assert B.traffic_from_profiles(rec["w_layout"]) == rec["bytes_per_launch"]
    # the counters cover ~1.01x the algorithmic bytes: no large re-read
    assert 1.0 <= rec["bytes_per_launch"] / rec["algorithmic_bytes_per_launch"] < 1.05
    assert B.traffic_from_profiles("rowmajor" if rec["w_layout"] == "tiled" else "tiled") is None
    monkeypatch.setattr(B, "sources_sha256", lambda: "0" * 64)
    assert B.traffic_from_profiles(rec["w_layout"]) is None

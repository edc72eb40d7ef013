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
    for cfg, name in B.TRAFFIC_RECORDS.items():
        path = os.path.join(ROOT, name)
        if not os.path.exists(path):
            continue
        rec = json.load(open(path))
        monkeypatch.setattr(B, "sources_sha256", lambda files, r=rec: r["source_sha256"])
        assert B.traffic_from_profiles(cfg, rec["w_layout"]) == rec["bytes_per_launch"]
        # the recorded bytes are the calibrated counters, and at least the
        # bytes the kernel must move
        cal = rec["copy_calibration"]
        want = (rec["fetch_size_kib_per_dispatch"] * 1024 * cal["fetch_factor"] +
                rec["write_size_kib_per_dispatch"] * 1024 * cal["write_factor"])
        assert abs(rec["bytes_per_launch"] - want) <= 1024
        assert rec["bytes_per_launch"] >= 0.95 * rec["algorithmic_bytes_per_launch"]
        other = "rowmajor" if rec["w_layout"] == "tiled" else "tiled"
        assert B.traffic_from_profiles(cfg, other) is None
        monkeypatch.setattr(B, "sources_sha256", lambda files: "0" * 64)
        assert B.traffic_from_profiles(cfg, rec["w_layout"]) is None
    assert B.traffic_from_profiles(99, "tiled") is None  # no record


def test_cpu_sample_keeps_weights_and_cuts_tokens():
    import types
    import numpy as np
    B = _bench()
    wl = types.SimpleNamespace(T=10, x=np.arange(40).reshape(10, 4), w1=np.ones(3))
    sub = B.token_sample(wl, 4)
    assert sub.T == 4 and sub.x.shape == (4, 4) and sub.w1 is wl.w1
    np.testing.assert_array_equal(sub.x, wl.x[:4])
    assert B.token_sample(wl, 10) is wl


def test_default_workload_is_the_prefill_layer():
    B = _bench()
    assert B.DEFAULT_CONFIG == 2

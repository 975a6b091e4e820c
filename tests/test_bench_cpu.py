"""bench.py host logic on the CPU: the one-GPU contract and the traffic figure's
guard (HBM bytes from committed counter runs are reported only while the kernel
sources they were measured on are unchanged)."""
import importlib.util
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one MI355X" in r.stderr and r.stdout == ""


def test_traffic_reported_only_for_the_measured_sources(tmp_path, monkeypatch):
    b = load_bench()
    src = tmp_path / "kernel.hip"
    src.write_text("// kernel v1\n")
    monkeypatch.setattr(b, "ROOT", str(tmp_path))
    monkeypatch.setattr(b, "KERNEL_SOURCES", ["kernel.hip"])
    traffic = tmp_path / "traffic.json"
    monkeypatch.setattr(b, "TRAFFIC_FILE", str(traffic))
    assert b.measured_traffic() is None  # no counter file
    traffic.write_text(json.dumps({"bytes_per_launch": 1234, "kernel_source_hash": b.kernel_source_hash()}))
    assert b.measured_traffic() == 1234
    src.write_text("// kernel v2\n")  # the kernel changed since the counters were taken
    assert b.measured_traffic() is None
    traffic.write_text("not json")
    assert b.measured_traffic() is None


def test_committed_traffic_file_names_the_dominant_kernel():
    with open(os.path.join(ROOT, "profiles", "attn_fwd_n75600_h10_traffic.json")) as f:
        t = json.load(f)
    assert t["kernel"] == "attn_fwd_kernel<128, 1, 8, 4, false, false, false, false>"
    # bytes = FETCH_SIZE * calibration + WRITE_SIZE, in KiB (the stored scale is rounded)
    want = (t["fetch_kib_per_dispatch"] * t["fetch_scale"] + t["write_kib_per_dispatch"] * t["write_scale"]) * 1024
    assert abs(t["bytes_per_launch"] - want) <= 1e-5 * want
    # at least the algorithmic bytes: q, k, V^T read and the output written (4 x 193.5 MB)
    assert t["bytes_per_launch"] >= 4 * 75600 * 10 * 128 * 2

"""Host-side logic of bench.py (no GPU): the one-GPU guard and the rule that the recorded
HBM traffic is reported only for the kernel source it was measured on."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def _traffic_file(tmp_path, digest, value=15250170):
    p = tmp_path / "traffic.txt"
    p.write_text("# comment = ignored\n"
                 f"traffic_bytes_per_launch = {value}\n"
                 "algorithmic_bytes_per_launch = 15052507\n"
                 f"source_sha256_16 = {digest}\n")
    return str(p)


def test_traffic_reported_for_the_measured_source(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", _traffic_file(tmp_path, bench.gemv_source_hash()))
    assert bench.measured_traffic() == 15250170


def test_traffic_dropped_when_the_source_changed(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", _traffic_file(tmp_path, "0" * 16))
    assert bench.measured_traffic() is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.txt"))
    assert bench.measured_traffic() is None


def test_committed_traffic_record_is_well_formed():
    kv = {}
    with open(os.path.join(ROOT, "profiles", "gemv_decode_step_m1_traffic.txt")) as f:
        for line in f:
            if "=" in line and not line.lstrip().startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    assert int(kv["algorithmic_bytes_per_launch"]) == 15052507
    # every weight byte read once; the activations re-read per workgroup add about 1 %
    assert 1.0 <= int(kv["traffic_bytes_per_launch"]) / 15052507 < 1.05
    assert len(kv["source_sha256_16"]) == 16

"""bench.py's command line on the host: a request for more than one GPU ends
with a message and exit status 2 before anything touches a GPU, and the
counter summary lookup keys on the kernel sources' hash and the workload."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_lookup_keys_on_source_hash_and_workload(tmp_path, monkeypatch):
    sha = bench.kernel_sha()
    assert len(sha) == 16 and int(sha, 16) >= 0
    f = tmp_path / "counters.txt"
    f.write_text(f"kernel_source_sha256_16: {sha}\nworkload: w1\nhbm_bytes_per_launch: 123456\n")
    monkeypatch.setattr(bench, "COUNTERS", str(f))
    assert bench.read_traffic("w1") == 123456
    assert bench.read_traffic("w2") is None                       # another workload
    f.write_text("kernel_source_sha256_16: 0000000000000000\nworkload: w1\nhbm_bytes_per_launch: 1\n")
    assert bench.read_traffic("w1") is None                       # taken from other kernel source

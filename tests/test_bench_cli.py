"""bench.py contract pieces that run without a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_multi_gpu_request_exits_with_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stdout


def test_workloads_match_synthetic_generator():
    sys.path.insert(0, ROOT)
    import bench
    from synthetic import WORKLOADS
    assert set(bench.WORKLOADS) == set(WORKLOADS)
    assert bench.WORKLOADS["low60s"]["preset"] == "low"

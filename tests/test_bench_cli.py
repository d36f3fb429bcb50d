"""bench.py's command line on the CPU: more than one GPU is refused with a
message (the path is built for one GPU), before any device is touched."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_unknown_workload_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "nope"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0 and "invalid choice" in r.stderr

"""Host-side checks of bench.py that need no GPU: a request for more than one
GPU is refused with a message (the path has no collective; one GPU's share
is the measured unit), and an unknown workload name is rejected."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_unknown_workload_is_rejected():
    r = run_bench("--workload", "no_such_workload")
    assert r.returncode != 0
    assert r.stdout == ""

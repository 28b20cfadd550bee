"""bench.py's command-line contract that holds without a GPU: more than one GPU is
refused with a message and exit status 2, before any device work."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_help_lists_the_workloads():
    r = subprocess.run([sys.executable, "bench.py", "--help"], cwd=ROOT, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0
    for opt in ("--steps", "--warmup", "--workload", "--paper", "--placements"):
        assert opt in r.stdout

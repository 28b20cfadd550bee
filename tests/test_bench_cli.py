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


def test_cpu_baseline_all_cores_timing():
    """The CPU baseline's all-cores leg on a small host workload: worker processes run the
    oracle's step on their requests and report their times (no GPU involved)."""
    sys.path.insert(0, ROOT)
    import bench
    from synth import workloads as SW
    wl = SW.direct_case(seed=5, B=5, L=1, Hq=8, Hkv=2, d=64, P=16, ctx=(100, 600))
    t1, tn, workers, per = bench.time_oracle(wl, wl.params, max_workers=2)
    assert workers == min(2, len(os.sched_getaffinity(0)), wl.B)
    assert len(per) == workers and all(p > 0 for p in per)
    assert t1 > 0 and tn >= max(per) * 0.5

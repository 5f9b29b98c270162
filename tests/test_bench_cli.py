"""bench.py's command line, checked on the CPU: one GPU only, and the step
counts it refuses (both exit before any device is touched)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_exits_with_a_message():
    r = run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_bad_step_counts_are_refused():
    for args in (["--steps", "0"], ["--warmup", "-1"]):
        r = run(*args)
        assert r.returncode == 2, args
        assert "--steps must be at least 1" in r.stderr and r.stdout == ""

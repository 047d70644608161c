"""bench.py on the host: argument handling that needs no GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_unknown_workload_is_rejected():
    r = run("--workload", "c9")
    assert r.returncode != 0
    assert "invalid choice" in r.stderr

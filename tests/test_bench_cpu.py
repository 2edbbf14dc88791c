"""The bench's command-line contract on the host: one GPU only, sane step counts.
These paths exit before any GPU work."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=300)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and not r.stdout.strip()


def test_bad_step_counts_are_refused():
    assert run("--steps", "0").returncode == 2
    assert run("--warmup", "-1").returncode == 2

"""bench.py's command-line contract, checked on the CPU: it measures one GPU
only, and refuses to run without one rather than falling back."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    res = run("--gpus", "2")
    assert res.returncode == 2
    assert "one GPU" in res.stderr


def test_help_lists_the_contract_flags():
    res = run("--help")
    assert res.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup", "--workload", "--b-layout", "--clock-seconds", "--no-vendor"):
        assert flag in res.stdout

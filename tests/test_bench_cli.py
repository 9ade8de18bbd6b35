"""bench.py's command-line contract on the CPU: one GPU only (--gpus N > 1
exits with status 2 and says why, before touching torch or the GPU), and the
help lists the measurement legs."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    for n in ("2", "8"):
        r = _run("--gpus", n)
        assert r.returncode == 2
        assert "one GPU" in r.stderr and r.stdout == ""


def test_help_lists_the_legs():
    r = _run("--help")
    assert r.returncode == 0
    for flag in ("--steps", "--warmup", "--gpus", "--multi", "--table", "--decode", "--no-cpu-baseline"):
        assert flag in r.stdout

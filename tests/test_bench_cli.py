"""bench.py's command line on the CPU: it measures one GPU only and says so for
any other count before touching a device; its modes are listed in --help."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_help_lists_the_modes():
    r = run("--help")
    assert r.returncode == 0
    for flag in ("--steps", "--warmup", "--all-configs", "--calibrate-copy", "--only"):
        assert flag in r.stdout

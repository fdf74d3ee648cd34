"""Command-line checks of bench.py that need no GPU: more than one GPU is
refused with a message before anything touches a device, and the options
parse."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_help_lists_the_timing_switches():
    r = _run("--help")
    assert r.returncode == 0
    for opt in ("--steps", "--warmup", "--no-graph", "--no-overlap", "--no-cpu-baseline",
                "--no-other-configs", "--copy-calibration-mib"):
        assert opt in r.stdout

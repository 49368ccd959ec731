"""The bench's command line on the host (no GPU is touched)."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_exits_with_a_message():
    r = run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr
    assert r.stdout == ""            # no JSON line


def test_help_lists_the_modes():
    r = run("--help")
    assert r.returncode == 0
    for flag in ("--workload", "--prefill", "--device-plan", "--graph", "--block-sparse", "--append",
                 "--event-every", "--ramp-ms", "--no-read-probe"):
        assert flag in r.stdout, flag


def test_graph_needs_a_device_plan():
    for args in (("--graph",), ("--graph", "--device-plan", "--block-sparse", "0.5")):
        r = run(*args)
        assert r.returncode == 2 and "--graph needs --device-plan" in r.stderr, args
        assert r.stdout == ""

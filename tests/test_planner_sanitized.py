"""The host planner under AddressSanitizer and UndefinedBehaviorSanitizer: planner.cpp
(plain C++17, no HIP) built with g++ and driven by tests/c/planner_sanitized.cpp over
3000 random and extreme batches; any sanitizer report or broken invariant fails."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_gqa_amd", "csrc")


def test_planner_is_clean_under_sanitizers(tmp_path):
    if shutil.which("g++") is None:
        pytest.skip("no g++")
    exe = str(tmp_path / "planner_sanitized")
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-I", CSRC, "-I", os.path.join(ROOT, "include"),
                    os.path.join(CSRC, "planner.cpp"), os.path.join(ROOT, "tests", "c", "planner_sanitized.cpp"),
                    "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip() == "ok 3000 plans" and "runtime error" not in r.stderr

"""The GEMM launch slicing (csrc/slices.h) keeps every 32-bit buffer offset and
buffer size of a launch within int32, tile overhang included, and covers every
row once (host code, checked on the CPU by tests/slices_check.cpp)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_launch_slices(tmp_path):
    exe = str(tmp_path / "slices_check")
    r = subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-fsanitize=undefined", "-fno-sanitize-recover=all",
                        os.path.join(ROOT, "tests", "slices_check.cpp"), "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr

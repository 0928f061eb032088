"""Host-side bounds check of the forward kernels' index arithmetic (CPU).

Builds tests/host/check_tiling.cpp with g++ against the same header the HIP
kernels include (csrc/fa_varlen_tiling.h) and runs it: every thread's buffer
load offsets against the resource extents, every LDS write/read index, and
the operand elements each MFMA lane reads."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "host", "check_tiling.cpp")
INC = os.path.join(ROOT, "variable_length_flashattention_cu_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_tiling_index_arithmetic(tmp_path):
    exe = str(tmp_path / "check_tiling")
    base = ["g++", "-std=c++17", "-O1", "-Wall", "-I", INC, SRC, "-o", exe]
    # host-only sanitizers when the toolchain has them
    r = subprocess.run(base + ["-fsanitize=address,undefined"], capture_output=True, text=True)
    if r.returncode != 0:
        r = subprocess.run(base, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "all tiling checks passed" in run.stdout

"""The C ABI from plain C: include/fa_varlen.h and include/fa_probe.h compile
as C99 with no HIP header (gcc -std=c99 -pedantic -Werror), link against the
in-tree libraries, and the calls in tests/host/abi_from_c.c return their
documented statuses on the host (every call there is answered before any
device work: sizes, tile heights, and validation failures)."""
import os
import shutil
import subprocess

import pytest

import variable_length_flashattention_cu_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "host", "abi_from_c.c")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_c_program_against_the_headers(tmp_path):
    libdir = os.path.dirname(fa.library_path())
    if not (os.path.exists(fa.library_path()) and os.path.exists(os.path.join(libdir, "libfa_probe.so"))):
        pytest.skip("libraries not built (run __graft_entry__.build())")
    exe = str(tmp_path / "abi_from_c")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
                    "-o", exe, SRC, "-L" + libdir, "-lfa_varlen", "-lfa_probe", "-Wl,-rpath," + libdir],
                   check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "C ABI checks passed" in r.stdout

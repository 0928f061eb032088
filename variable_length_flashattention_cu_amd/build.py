"""Build libfa_varlen.so in place with hipcc for gfx950.

    python -m variable_length_flashattention_cu_amd.build [--asm DIR]

The library is written next to this file (the package directory), so it
travels with the source tree.  ``--asm DIR`` also writes the device assembly
of the kernels to DIR for inspection.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libfa_varlen.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
# measurement aid (include/fa_probe.h): the matrix-core ceiling probe
PROBE_PATH = os.path.join(PKG_DIR, "libfa_probe.so")
PROBE_SOURCES = [os.path.join(CSRC, "fa_probe.hip")]

SOURCES = [os.path.join(CSRC, "fa_varlen_kernels.hip"), os.path.join(CSRC, "fa_varlen_bwd.hip"),
           os.path.join(CSRC, "fa_varlen_decode.hip"), os.path.join(CSRC, "fa_varlen_scratch.hip"),
           os.path.join(CSRC, "fa_varlen_api.cpp")]
ARCH = "gfx950"
# Packed fp32 VALU forms are kept out of the generated code.
NO_PACKED_FP32 = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Per-source code generation options.  The backward kernel keeps its matrix
# accumulators in architectural VGPRs: with accumulation registers the
# allocator moved the dK/dV accumulators out and back every step to make room
# for the score tiles.
SOURCE_FLAGS = {"fa_varlen_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def common_flags():
    return ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-I", INCLUDE, "-I", CSRC,
            "-Wall", "-Wno-unused-function"] + NO_PACKED_FP32


def source_flags(src: str) -> list:
    return SOURCE_FLAGS.get(os.path.basename(src), [])


def run(cmd: list, verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")


def build(verbose: bool = False, asm_dir: str | None = None) -> str:
    """Build libfa_varlen.so and libfa_probe.so; returns the attention library's path."""
    _link(LIB_PATH, SOURCES, verbose)
    _link(PROBE_PATH, PROBE_SOURCES, verbose)
    if asm_dir:
        os.makedirs(asm_dir, exist_ok=True)
        for src in SOURCES + PROBE_SOURCES:
            if src.endswith(".hip"):
                asm = os.path.join(asm_dir, os.path.basename(src)[:-4] + ".s")
                cmd = [hipcc()] + common_flags() + source_flags(src) + ["--cuda-device-only", "-S", "-o", asm, src]
                subprocess.run(cmd, check=True, capture_output=True, text=True)
    return LIB_PATH


def _link(lib_path: str, sources: list, verbose: bool) -> None:
    tmp = lib_path + ".tmp"
    objs = []
    procs = []
    for src in sources:  # one object per source (own options), compiled in parallel
        obj = lib_path + "." + os.path.basename(src) + ".o"
        cmd = [hipcc()] + common_flags() + source_flags(src) + ["-c", "-o", obj, src]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True), obj))
    failed = False
    for proc, obj in procs:
        out, err = proc.communicate()
        if proc.returncode != 0:
            sys.stderr.write(out + err)
            failed = True
        objs.append(obj)
    if failed:
        raise RuntimeError("hipcc failed")
    run([hipcc()] + common_flags() + ["-shared", "-o", tmp] + objs, verbose)
    for obj in objs:
        os.remove(obj)
    os.replace(tmp, lib_path)


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", default=None, help="also write device assembly to this directory")
    ap.add_argument("-q", "--quiet", action="store_true")
    args = ap.parse_args()
    path = build(verbose=not args.quiet, asm_dir=args.asm)
    print(path)


if __name__ == "__main__":
    main()

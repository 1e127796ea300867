"""Build libsketchssm.so in-tree (hipcc for gfx950; the host planner with g++).

    python -m rank_state_read_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libsketchssm.so")
BUILD_DIR = os.path.join(PKG, "_build")

HIP_SOURCES = ["read.hip", "flush.hip", "rmw.hip", "stream.hip"]
CXX_SOURCES = ["plan.cpp"]

# Packed-fp32 VALU forms are kept out of the generated code.
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"build step failed: {' '.join(cmd)}")
    if verbose and (r.stdout or r.stderr):
        sys.stderr.write(r.stdout + r.stderr)


def build(verbose: bool = False, save_temps: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    hipcc = _hipcc()
    inc = [f"-I{INCLUDE}", f"-I{CSRC}"]
    objs = []
    for src in CXX_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        _run(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-c", os.path.join(CSRC, src),
              "-o", obj] + inc, verbose)
        objs.append(obj)
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        extra = ["-save-temps=obj"] if save_temps else []
        _run([hipcc] + HIP_FLAGS + extra + ["-c", os.path.join(CSRC, src), "-o", obj] + inc, verbose)
        objs.append(obj)
    tmp = OUT + ".tmp"
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs, verbose)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, save_temps="--save-temps" in sys.argv))

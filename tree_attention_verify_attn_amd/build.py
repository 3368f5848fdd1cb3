"""Compile libtreeattn.so (HIP, gfx950) in-tree, and the measurement library
libtafloor.so beside it.

The attention library is one translation unit (csrc/ta_api.hip includes the
kernels); the measurement library holds only the plain streaming-read kernel
that the benchmark's floor mode times (floor/floor_read.hip, kept out of csrc/
so that the attention kernels' source hash does not cover it).  Both are built
with hipcc for gfx950 only.  Packed-fp32 instruction selection is disabled for
all device code.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO_DIR = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(REPO_DIR, "include")
LIB_PATH = os.path.join(PKG_DIR, "libtreeattn.so")
FLOOR_LIB_PATH = os.path.join(PKG_DIR, "libtafloor.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # kernels whose leading arguments are scalars get them in SGPRs with the
    # dispatch (at most 16 dwords) instead of by a load at entry
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-Wall",
    "-Wno-unused-command-line-argument",
]


def sources():
    return [os.path.join(CSRC, "ta_api.hip")]


def build_library(out: str = LIB_PATH, verbose: bool = False, srcs=None) -> str:
    """Build the shared library to ``out`` (atomically replaced) and return its path."""
    tmp = out + f".tmp{os.getpid()}"
    cmd = [HIPCC, *FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", *(srcs or sources()), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature flag; drop that noise
    noise = ("packed-fp32-ops", "not a recognized feature for this target")
    err = "\n".join(l for l in res.stderr.splitlines() if not any(n in l for n in noise))
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, out)
    return out


def build_floor_library(out: str = FLOOR_LIB_PATH, verbose: bool = False) -> str:
    """Build the measurement library (streaming-read floor kernel) to ``out``."""
    return build_library(out, verbose, [os.path.join(PKG_DIR, "floor", "floor_read.hip")])


if __name__ == "__main__":
    print(build_library(verbose=True))
    print(build_floor_library(verbose=True))

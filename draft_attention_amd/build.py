"""Compile libdraft_attn.so in-tree for gfx950 with hipcc.

Usage: python draft_attention_amd/build.py  (or __graft_entry__.build()). It does
not import the package, whose import loads the library this script builds.
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libdraft_attn.so")
BUILD_DIR = os.path.join(HERE, "_build")
HIP_SOURCES = [os.path.join(HERE, "csrc", n) for n in ("decode.hip", "append.hip", "draft.hip")]
CXX_SOURCES = [os.path.join(HERE, "csrc", "host.cpp")]  # pure C++: built by the host compiler

# Packed fp32 VALU ops are turned off for all device code. Kernel-argument
# preloading: a kernel's leading scalar arguments (up to 16 dwords) arrive in
# registers when its waves start, instead of through a memory read.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-mllvm", "-amdgpu-kernarg-preload-count=16",
             "-Wall", "-Wno-unused-command-line-argument"]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(ln for ln in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in ln)
    if res.returncode != 0:
        sys.stderr.write(out + "\n")
        raise RuntimeError(f"{cmd[0]} failed with status {res.returncode}")
    if verbose and out.strip():
        print(out)
    elif res.returncode == 0 and "error" in out.lower():
        sys.stderr.write(out + "\n")


def build(verbose: bool = False, extra=()) -> str:
    """Compile every source and link libdraft_attn.so next to this file."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    cxx = os.environ.get("CXX", "g++")
    os.makedirs(BUILD_DIR, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include")]
    objs = []
    for src in CXX_SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        _run([cxx, *CXX_FLAGS, *inc, "-c", src, "-o", obj], verbose)
        objs.append(obj)
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        _run([hipcc, *HIP_FLAGS, *extra, *inc, "-c", src, "-o", obj], verbose)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

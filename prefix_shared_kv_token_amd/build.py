"""Builds librdx.so in-tree for gfx950 (hipcc for the HIP sources, g++ for
the host-only C++), so the library travels with the source tree."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "librdx.so")

HOST_SOURCES = ["radix_tree.cpp", "plan.cpp", "schedule.cpp", "prefix_groups.cpp", "token_batch.cpp", "job.cpp", "capi_host.cpp"]
HIP_SOURCES = ["device.hip"]
ARCH = os.environ.get("RDX_OFFLOAD_ARCH", "gfx950")
# packed fp32 instructions are disabled for all device code
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-Wno-unused-parameter"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("build step failed: " + " ".join(cmd))
    return r


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    inc = ["-I", INCLUDE, "-I", CSRC]
    objs = []
    for s in HOST_SOURCES:
        o = os.path.join(BUILD, s + ".o")
        _run(["g++", *HOST_FLAGS, *inc, "-c", os.path.join(CSRC, s), "-o", o])
        objs.append(o)
    for s in HIP_SOURCES:
        o = os.path.join(BUILD, s + ".o")
        _run(["hipcc", *HIP_FLAGS, *inc, "-c", os.path.join(CSRC, s), "-o", o])
        objs.append(o)
    tmp = LIB + ".tmp"
    _run(["hipcc", "-shared", f"--offload-arch={ARCH}", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)

"""Builds librdx.so in-tree for gfx950 (hipcc for the HIP sources, g++ for
the host-only C++), so the library travels with the source tree."""
from __future__ import annotations

import os
import re
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
# the compiler reports each kernel's registers, scratch and LDS
RESOURCE_REMARKS = ["-Rpass-analysis=kernel-resource-usage"]
RESOURCES = os.path.join(BUILD, "kernel_resources.txt")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("build step failed: " + " ".join(cmd))
    return r


def kernel_resources(remarks: str) -> dict:
    """Per kernel (mangled name): the resource fields of the compiler's
    kernel-resource-usage remarks (VGPRs, AGPRs, ScratchSize, Occupancy,
    LDS Size, ...), as integers where they are numbers."""
    out, cur = {}, None
    for line in remarks.splitlines():
        m = re.search(r"remark:\s+Function Name: (\S+)", line)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z][A-Za-z ]*?)(?: \[[^\]]*\])?: (\S+) \[-Rpass-analysis", line)
        if m and cur is not None:
            v = m.group(2)
            cur[m.group(1)] = int(v) if v.isdigit() else v
    return out


def check_resources(res: dict) -> None:
    """Every kernel must run without scratch memory: a spill or a private
    array lowered to scratch slows a kernel several-fold without changing
    its results (a select of two vectors in the 64-bit decode path once did:
    4.5x slower), so the build fails instead."""
    bad = {k: v.get("ScratchSize") for k, v in res.items() if v.get("ScratchSize", 0) != 0}
    if bad:
        raise RuntimeError("kernels using scratch memory (bytes per lane): " + repr(bad))


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    inc = ["-I", INCLUDE, "-I", CSRC]
    objs = []
    for s in HOST_SOURCES:
        o = os.path.join(BUILD, s + ".o")
        _run(["g++", *HOST_FLAGS, *inc, "-c", os.path.join(CSRC, s), "-o", o])
        objs.append(o)
    res = {}
    for s in HIP_SOURCES:
        o = os.path.join(BUILD, s + ".o")
        r = _run(["hipcc", *HIP_FLAGS, *RESOURCE_REMARKS, *inc, "-c", os.path.join(CSRC, s), "-o", o])
        res.update(kernel_resources(r.stderr))
        objs.append(o)
    with open(RESOURCES, "w") as f:
        for k in sorted(res):
            f.write(k + " " + " ".join(f"{n}={v}" for n, v in res[k].items()) + "\n")
    if not res:
        raise RuntimeError("no kernel resource remarks from the compiler")
    check_resources(res)
    tmp = LIB + ".tmp"
    _run(["hipcc", "-shared", f"--offload-arch={ARCH}", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)

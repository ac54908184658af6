"""Builds librdx_host_san.so: the host C++ of librdx (tree, planner,
ordering, batching, prefix groups, job runner, C ABI) with AddressSanitizer
and UndefinedBehaviorSanitizer, plus host-only stand-ins that make every
device entry point fail with RDX_EUNSUPPORTED.  CPU only: it compiles no
HIP code.  Run the CPU test suite against it with

    python prefix_shared_kv_token_amd/sanitize/build_host_san.py
    RDX_LIB=prefix_shared_kv_token_amd/sanitize/librdx_host_san.so \\
    LD_PRELOAD="$(g++ -print-file-name=libasan.so)${LD_PRELOAD:+:$LD_PRELOAD}" \\
    ASAN_OPTIONS=detect_leaks=0 UBSAN_OPTIONS=halt_on_error=1:print_stacktrace=1 \\
    python -m pytest tests -q -m "not gpu"

(the Python interpreter is not instrumented, so the ASan runtime is
preloaded; leak checking is off because the interpreter keeps its own
allocations to the end).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "librdx_host_san.so")
SOURCES = [os.path.join(CSRC, s) for s in
           ("radix_tree.cpp", "plan.cpp", "schedule.cpp", "prefix_groups.cpp", "token_batch.cpp", "job.cpp",
            "capi_host.cpp")] + [os.path.join(HERE, "host_only.cpp")]
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
FLAGS = ["-O1", "-g", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build() -> str:
    os.makedirs(BUILD, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs = []
    for s in SOURCES:
        o = os.path.join(BUILD, os.path.basename(s) + ".o")
        subprocess.run(["g++", *FLAGS, *SAN, *inc, "-c", s, "-o", o], check=True)
        objs.append(o)
    subprocess.run(["g++", "-shared", *SAN, "-Wl,--no-undefined", *objs, "-o", LIB], check=True)
    return LIB


if __name__ == "__main__":
    print(build())

"""Prefix-shared paged-KV attention (the RadixAttention data path) on MI355X.

librdx.so (built from csrc/) holds the radix tree, the batch planner and the
gfx950 kernels; `rdx` is its ctypes binding, `runtime.Runtime` the serving
loop over it, `driver.WorkloadRun` the phase driver for synthetic workloads.
"""
from . import rdx  # noqa: F401

__all__ = ["rdx"]

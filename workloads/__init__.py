"""Seeded synthetic inputs shared by the GPU path's tests/bench and by the oracle.

This package only *draws inputs*: token ids, query/key/value tensors and the
shape of the sharing tree (which request carries which token segments).  It
holds none of the method's arithmetic (no matching, no allocation, no
attention); both the HIP path and the oracle consume what it produces.
"""
from .configs import CONFIGS, Config, config_by_name
from .gen import Workload, Request, Phase, bf16_round_bits, bf16_bits_to_f32
from .queue import waiting_queue, decode_lengths, reuse_stream

__all__ = [
    "CONFIGS", "Config", "config_by_name", "Workload", "Request", "Phase",
    "bf16_round_bits", "bf16_bits_to_f32", "waiting_queue", "decode_lengths", "reuse_stream",
]

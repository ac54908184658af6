"""Seeded request-level inputs: waiting queues (a workload's prompts in a
random arrival order) and per-request output lengths.  No scheduling logic
here; the code under test and the oracle both consume the same draws."""
from __future__ import annotations

import numpy as np

from .gen import SEED, Workload

TAG_QUEUE = 9
TAG_DLEN = 10


def waiting_queue(wl: Workload, n: int, seed: int = 0) -> list:
    """`n` leaf prompts of `wl` (int32 arrays), drawn without replacement, in a
    seeded random arrival order."""
    rng = np.random.default_rng(np.random.SeedSequence([SEED, wl.cfg.index, TAG_QUEUE, seed]))
    leaves = wl.leaf_requests
    pick = rng.choice(len(leaves), size=min(n, len(leaves)), replace=False)
    return [wl.prompt_tokens(leaves[int(i)]) for i in pick]


def decode_lengths(wl: Workload, seed: int = 0) -> np.ndarray:
    """Per leaf request, how many of its `decode_steps` drawn tokens it
    generates: seeded uniform in [1, decode_steps] (outputs of varied
    length, as a serving job sees them)."""
    rng = np.random.default_rng(np.random.SeedSequence([SEED, wl.cfg.index, TAG_DLEN, seed]))
    t = wl.cfg.decode_steps
    n = len(wl.leaf_requests)
    return rng.integers(1, t + 1, size=n).astype(np.int32) if t > 0 else np.zeros(n, np.int32)

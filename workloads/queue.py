"""Seeded waiting queues for the request-ordering measurements: prompts of a
workload's sharing tree arriving in a random order (no ordering logic here;
the scheduler under test and the oracle both consume the same queue)."""
from __future__ import annotations

import numpy as np

from .gen import SEED, Workload

TAG_QUEUE = 9


def waiting_queue(wl: Workload, n: int, seed: int = 0) -> list:
    """`n` leaf prompts of `wl` (int32 arrays), drawn without replacement, in a
    seeded random arrival order."""
    rng = np.random.default_rng(np.random.SeedSequence([SEED, wl.cfg.index, TAG_QUEUE, seed]))
    leaves = wl.leaf_requests
    pick = rng.choice(len(leaves), size=min(n, len(leaves)), replace=False)
    return [wl.prompt_tokens(leaves[int(i)]) for i in pick]

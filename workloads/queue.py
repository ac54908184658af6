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


def reuse_stream(n: int = 400, seed: int = 0, hot=(1000, 1000, 1000, 1000), weights=(8, 4, 2, 1),
                 question: int = 40, one_off: int = 1500, p_hot: float = 0.5, vocab: int = 32000):
    """A request stream that puts a cache under eviction pressure: with
    probability p_hot a request reuses one of the `hot` system prompts
    (chosen by `weights`) followed by `question` fresh tokens, else it is a
    one-off prompt of `one_off` fresh tokens.  -> (prompts, is_hot), in
    arrival order; hot prompts differ in their first token."""
    rng = np.random.default_rng(np.random.SeedSequence([SEED, 99, TAG_QUEUE, seed]))
    firsts = rng.choice(vocab, size=len(hot), replace=False)
    prefixes = []
    for f, length in zip(firsts, hot):
        p = rng.integers(0, vocab, size=length).astype(np.int32)
        p[0] = f
        prefixes.append(p)
    w = np.asarray(weights, np.float64) / np.sum(weights)
    prompts, is_hot = [], []
    for _ in range(n):
        if rng.random() < p_hot:
            k = int(rng.choice(len(hot), p=w))
            prompts.append(np.concatenate([prefixes[k], rng.integers(0, vocab, size=question).astype(np.int32)]))
            is_hot.append(True)
        else:
            prompts.append(rng.integers(0, vocab, size=one_off).astype(np.int32))
            is_hot.append(False)
    return prompts, np.array(is_hot)

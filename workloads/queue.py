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


TAG_SERVE = 11


def served_queue(seed: int = 0, system=(300, 180, 120), popularity=(5, 3, 2), one_offs: int = 4,
                 one_off_len=(150, 260), suffix_len=(16, 64), decode_steps: int = 4, vocab: int = 32000):
    """A waiting queue for an end-to-end serving run: popularity[i] requests
    reuse system prompt i (lengths `system`) followed by a fresh suffix, and
    `one_offs` requests are fresh prompts; seeded random arrival order.
    Every prompt is a list of logical segments (id, length), so K/V can be
    drawn per segment: system prompt i is segment i, request j's own part is
    segment len(system) + j, its generated tokens segment 10000 + j.
    First tokens of sibling segments are distinct (system prompts and
    one-offs among each other; suffixes of one system prompt among each
    other), so the tree the prompts build is exactly the intended one.
    -> (prompts, segments, generated, hot) in arrival order; hot[j] marks the
    requests that reuse a system prompt."""
    rng = np.random.default_rng(np.random.SeedSequence([SEED, 98, TAG_SERVE, seed]))
    n_sys = len(system)
    n_req = int(sum(popularity)) + one_offs
    firsts = rng.choice(vocab, size=n_sys + one_offs, replace=False)
    sys_tok = []
    for i, length in enumerate(system):
        t = rng.integers(0, vocab, size=length).astype(np.int32)
        t[0] = firsts[i]
        sys_tok.append(t)
    kinds = [i for i, c in enumerate(popularity) for _ in range(c)] + [-1] * one_offs
    suffix_firsts = rng.choice(vocab, size=n_req, replace=False)
    prompts, segments, generated, hot = [], [], [], []
    n_one = 0
    for j, kind in enumerate(kinds):
        if kind >= 0:
            own = rng.integers(0, vocab, size=int(rng.integers(suffix_len[0], suffix_len[1] + 1))).astype(np.int32)
            own[0] = suffix_firsts[j]
            prompts.append(np.concatenate([sys_tok[kind], own]))
            segments.append([(kind, len(sys_tok[kind])), (n_sys + j, len(own))])
        else:
            own = rng.integers(0, vocab, size=int(rng.integers(one_off_len[0], one_off_len[1] + 1))).astype(np.int32)
            own[0] = firsts[n_sys + n_one]
            n_one += 1
            prompts.append(own)
            segments.append([(n_sys + j, len(own))])
        generated.append(rng.integers(0, vocab, size=decode_steps).astype(np.int32))
        hot.append(kind >= 0)
    order = rng.permutation(n_req)
    return ([prompts[i] for i in order], [segments[i] for i in order],
            [(10000 + int(i), generated[i]) for i in order], np.array([hot[i] for i in order]))


def segment_values(seg: int, length: int, heads: int, head_dim: int, sigma: float, tag: int, seed: int = 0):
    """N(0,1)*sigma float32 [length, heads, head_dim] of one logical segment
    (tag: 0 K, 1 V, 2 Q), seeded by the segment id."""
    rng = np.random.default_rng(np.random.SeedSequence([SEED, 98, TAG_SERVE, seed, tag, seg]))
    return (rng.standard_normal((length, heads, head_dim), dtype=np.float32) * np.float32(sigma))

"""Throughput-oriented token batching (oracle; test infrastructure only: tests,
the smoke check and the benchmark's CPU leg import it, never the product).

Passages followed (BatchLLM explainer):
  * Throughput-oriented Token Batching, Equations 3-4: requests sharing a
    prefix are scheduled as a group; groups with a higher decoding ratio go
    first, the group ratio taking the output length as 1, i.e. one over the
    group's prefill tokens (common prefix + every distinct prompt);
  * three-queue fetching: every iteration takes tokens from the decoding
    queue first (one token per request already decoding), then the
    distinct-prompt queue (requests whose common prefix is processed), then
    the common-prefix queue (prefixes of groups not yet prefilled);
  * Memory-centric Token Batching: an iteration's batch is bounded by the KV
    memory it needs, not by a request count.  Read here as: every decoding
    request's token is in the batch; the prefill chunks (at most s_chunk
    tokens each, two KV entries per token) come from the head of the queue,
    as many as fit beside the memory the decoding requests hold under
    M_threshold.

Readings of points the pages leave open (the product follows the same):
  * R_group = 1 / (L_prefix + sum of L_distinct) as printed: groups run in
    ascending order of prefill tokens, ties by group index;
  * the decoding requests' KV memory counts what they hold: a group's common
    prefix once (it is shared, the point of prefix sharing), plus each
    decoding request's distinct prompt and the tokens it generated so far,
    before this iteration's token; decode tokens are always taken and add no
    memory in that iteration; requests still in prefill are not counted;
  * a pending chunk is the next min(s_chunk, remaining) tokens of one
    request's distinct prompt or of one group's prefix; at most one chunk per
    pending item per iteration; the chunks taken are a head of the queue (a
    chunk that does not fit ends the batch; later, smaller ones are not
    tried);
  * a distinct prompt enters the queue the iteration after its group's
    prefix is complete (immediately if the prefix is empty); a request
    decodes from the iteration after its prompt is complete and generates
    `decode` tokens, the t-th at position L_prefix + L_distinct + t;
  * queue order within a queue follows the group order, then the request's
    index in its group;
  * M_threshold >= 2 s_chunk, so an iteration with nothing decoding always
    takes one chunk (progress).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

DECODE, DISTINCT, PREFIX = 0, 1, 2


@dataclass(frozen=True)
class Group:
    prefix_len: int
    distinct: tuple   # distinct prompt length of each member (>= 1)
    decode: tuple     # tokens each member generates (>= 0)


def group_order(groups) -> list:
    """Descending R_group = 1 / (prefix + sum distinct), ties by index."""
    return sorted(range(len(groups)), key=lambda g: (groups[g].prefix_len + sum(groups[g].distinct), g))


def batch_iterations(groups, s_chunk: int, m_threshold: int) -> list:
    """Runs the whole job -> list of iterations, each a list of entries
    (kind, group, member, begin, count): `begin` is the position of the
    entry's first token in its sequence (the prefix for PREFIX entries,
    prefix + distinct + generated for the member's own tokens), member = -1
    for PREFIX entries.  Entries: decode tokens first, then the chunks in
    queue order."""
    if s_chunk < 1 or m_threshold < 2 * s_chunk:
        raise ValueError("need s_chunk >= 1 and m_threshold >= 2 * s_chunk")
    for g in groups:
        if len(g.distinct) != len(g.decode) or len(g.distinct) == 0:
            raise ValueError("every group needs members, each with a distinct length and a decode length")
        if g.prefix_len < 0 or min(g.distinct) < 1 or min(g.decode) < 0:
            raise ValueError("prefix >= 0, distinct >= 1, decode >= 0")
    order = group_order(groups)
    pre_done = {g: 0 for g in order}
    pre_complete_at = {g: (-1 if groups[g].prefix_len == 0 else None) for g in order}
    dist_done = {(g, j): 0 for g in order for j in range(len(groups[g].distinct))}
    prompt_complete_at = {}
    generated = {k: 0 for k in dist_done}
    iterations = []
    it = 0
    while True:
        # requests decoding at the start of this iteration
        decoding = [(g, j) for g in order for j in range(len(groups[g].distinct))
                    if (g, j) in prompt_complete_at and prompt_complete_at[(g, j)] < it
                    and generated[(g, j)] < groups[g].decode[j]]
        pending = []  # (kind, g, j, remaining, begin)
        for g in order:
            if pre_complete_at[g] is not None and pre_complete_at[g] < it:
                for j, ld in enumerate(groups[g].distinct):
                    if dist_done[(g, j)] < ld:
                        pending.append((DISTINCT, g, j, ld - dist_done[(g, j)], groups[g].prefix_len + dist_done[(g, j)]))
        for g in order:
            if pre_done[g] < groups[g].prefix_len:
                pending.append((PREFIX, g, -1, groups[g].prefix_len - pre_done[g], pre_done[g]))
        if not decoding and not pending:
            break
        # KV entries (K and V: two per token) the decoding requests hold
        held = 2 * (sum(groups[g].prefix_len for g in {g for g, _ in decoding})
                    + sum(groups[g].distinct[j] + generated[(g, j)] for g, j in decoding))
        # the batch is bounded by KV memory: the chunks taken are the longest
        # head of the pending queue whose entries, added to what is held,
        # stay within M_threshold
        sizes = [min(s_chunk, remaining) for _, _, _, remaining, _ in pending]
        need = np.cumsum(2 * np.asarray(sizes, dtype=np.int64)) if sizes else np.zeros(0, np.int64)
        n_take = int(np.searchsorted(need, m_threshold - held, side="right"))
        batch = [(DECODE, g, j, groups[g].prefix_len + groups[g].distinct[j] + generated[(g, j)], 1)
                 for g, j in decoding]
        batch += [(kind, g, j, begin, c) for (kind, g, j, _, begin), c in zip(pending[:n_take], sizes)]
        assert batch, "no progress"
        for kind, g, j, begin, c in batch:
            if kind == DECODE:
                generated[(g, j)] += 1
            elif kind == DISTINCT:
                dist_done[(g, j)] += c
                if dist_done[(g, j)] == groups[g].distinct[j]:
                    prompt_complete_at[(g, j)] = it
            else:
                pre_done[g] += c
                if pre_done[g] == groups[g].prefix_len:
                    pre_complete_at[g] = it
        iterations.append(batch)
        it += 1
    return iterations

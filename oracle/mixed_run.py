"""A two-level workload as one token-batched job, through the oracle's cache
model (test infrastructure only).

The iterations come from token_batching.batch_iterations (groups = the
top-level prefixes, members = the leaf requests under each).  Cache calls
per iteration, the same sequence the product's mixed runner makes:
  1. admissions, in entry order: a group's prefix request at its first
     prefix chunk, a member at its first distinct chunk -- match_prefix of
     the prompt, lock the node, alloc(prompt - matched) for the row;
  2. one alloc(number of decode entries); the ascending slots go to the
     decode entries in order, at their positions;
  3. the attention of the batch (its values do not depend on the batching:
     a token at position p attends to positions 0..p of its sequence, so the
     expected outputs are those of request_attention);
  4. the requests whose last token was in the batch, in entry order:
     insert(sequence, row), free the duplicates row[matched:present),
     unlock.
"""
from __future__ import annotations

import numpy as np

from .cache_model import TokenTrieCache
from .run import request_attention
from .token_batching import DECODE, DISTINCT, PREFIX, Group, batch_iterations


def mixed_groups(wl, decode_len=None):
    """(groups, member requests per group) of a two-level workload;
    decode_len: tokens each leaf request generates (in leaf order; all of its
    decode_steps by default)."""
    pre, mem = wl.phases[0].requests, wl.phases[1].requests
    tlen = {r.rid: (r.decode_steps if decode_len is None else int(decode_len[i])) for i, r in enumerate(mem)}
    by_node = {r.node: g for g, r in enumerate(pre)}
    members = [[] for _ in pre]
    for r in mem:
        members[by_node[r.path[0]]].append(r)
    groups = [Group(p.own_len, tuple(r.own_len for r in ms), tuple(tlen[r.rid] for r in ms))
              for p, ms in zip(pre, members)]
    return groups, members


def run_mixed(wl, s_chunk: int, m_threshold: int, decode_len=None, num_slots: int | None = None):
    """-> dict with the iterations, and per request (rid) its matched length
    and final page-table row."""
    cfg = wl.cfg
    groups, members = mixed_groups(wl, decode_len)
    tlen = {r.rid: t for g, ms in zip(groups, members) for r, t in zip(ms, g.decode)}
    pre = wl.phases[0].requests
    its = batch_iterations(groups, s_chunk, m_threshold)
    cache = TokenTrieCache(num_slots or cfg.total_tokens())
    state = {}  # rid -> [matched, node, row]
    matched, rows = {}, {}

    def request(kind, g, j):
        return pre[g] if kind == PREFIX else members[g][j]

    for batch in its:
        for kind, g, j, begin, c in batch:
            start = (kind == PREFIX and begin == 0) or (kind == DISTINCT and begin == groups[g].prefix_len)
            if start:
                r = request(kind, g, j)
                prompt = wl.prompt_tokens(r)
                m, slots, node = cache.match_prefix(prompt)
                cache.lock(node)
                state[r.rid] = [m, node, list(slots) + cache.alloc(len(prompt) - m)]
                matched[r.rid] = m
        dec = [(g, j) for kind, g, j, _, _ in batch if kind == DECODE]
        if dec:
            for (g, j), s in zip(dec, cache.alloc(len(dec))):
                state[members[g][j].rid][2].append(s)
        for kind, g, j, begin, c in batch:
            r = request(kind, g, j)
            end = begin + c
            t = tlen.get(r.rid, 0)
            if end == r.prompt_len + t:
                m, node, row = state.pop(r.rid)
                seq = np.concatenate([wl.prompt_tokens(r), wl.decode_tokens(r)[:t]]) if t else wl.prompt_tokens(r)
                k, _ = cache.insert(seq, row)
                cache.free(row[m:k])
                cache.unlock(node)
                rows[r.rid] = np.asarray(row, np.int32)
    assert not state, "requests left unfinished"
    return {"iterations": its, "matched": matched, "rows": rows, "stats": cache.stats()}


def expected_outputs(wl, rids=None):
    """rid -> float64 [tokens the request computes, Hq, D]: its own prompt
    tokens, then all of its drawn decode tokens (the prefix request: the
    prefix).  A request generating fewer tokens computes a leading part."""
    out = {}
    for r in wl.phases[0].requests + wl.phases[1].requests:
        if rids is not None and r.rid not in rids:
            continue
        e, d = request_attention(wl, r)
        out[r.rid] = np.concatenate([e, d]) if len(d) else e
    return out

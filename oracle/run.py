"""Drive a synthetic workload through the oracle (test infrastructure only).

Serving protocol (the same sequence of cache calls the product's runtime
makes; the SGLang paper notes, section 3, describe the frontend hint: on a
fork the shared prefix is sent first so the tree exists before the branches
arrive):

  for each extend phase, requests in order:
      admit:   m, slots, node = match_prefix(prompt); lock(node);
               page-table row = slots + alloc(len(prompt) - m)
      extend:  the request's queries are its tokens at positions m..n-1
  leaf phase only, for each decode step t:
      one alloc(R) call; the R ascending slots go to the leaf requests in order
      and each new token (position n + t) attends to positions 0..n+t
  finish (requests in order):
      k, _ = insert(prompt + decode tokens, row); free(row[m:k]); unlock(node)

Saved tokens are the matched lengths; N_processed counts every extend
request's computed tokens (hints included), N_logical the leaf requests'
prompt lengths (hint requests are not logical requests).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .attention import causal_attention
from .cache_model import TokenTrieCache
from .saving import r_saving, hit_rate


@dataclass
class OracleResult:
    matched: dict = field(default_factory=dict)      # rid -> m
    node: dict = field(default_factory=dict)         # rid -> node id returned by match
    rows: dict = field(default_factory=dict)         # rid -> np.int32 page-table row
    present: dict = field(default_factory=dict)      # rid -> present length at insert
    extend_out: dict = field(default_factory=dict)   # rid -> float64 [own_len, Hq, D]
    decode_out: dict = field(default_factory=dict)   # rid -> float64 [T, Hq, D]
    n_processed: int = 0
    n_logical: int = 0
    r_saving: float = 0.0
    hit_rate: float = 0.0
    stats: dict = field(default_factory=dict)


def request_attention(wl, req):
    """Oracle outputs of one request: (extend [own_len, Hq, D], decode [T, Hq, D])."""
    k, v = wl.request_full_kv(req)
    q_parts = [wl.request_q(req)]
    pos = list(range(req.prompt_len - req.own_len, req.prompt_len))
    if req.decode_steps:
        q_parts.append(wl.decode_q(req))
        pos += list(range(req.prompt_len, req.prompt_len + req.decode_steps))
    o = causal_attention(np.concatenate(q_parts), k, v, np.asarray(pos))
    return o[: req.own_len], o[req.own_len:]


def run_workload(wl, num_slots: int | None = None, attention_for=None, match_unit: int = 1, prepare=None):
    """attention_for: None = every request, an iterable of rids, or () for none.
    prepare: optional callable applied to the fresh cache before the phases
    (e.g. allocations that fragment the pool)."""
    cfg = wl.cfg
    cache = TokenTrieCache(num_slots or cfg.total_tokens(), match_unit)
    if prepare is not None:
        prepare(cache)
    res = OracleResult()
    want = None if attention_for is None else set(attention_for)
    n_phases = len(wl.phases)
    for pi, phase in enumerate(wl.phases):
        leaf = pi == n_phases - 1
        admitted = []
        for req in phase.requests:
            prompt = wl.prompt_tokens(req)
            m, slots, node = cache.match_prefix(prompt)
            cache.lock(node)
            row = list(slots) + cache.alloc(len(prompt) - m)
            res.matched[req.rid] = m
            res.node[req.rid] = node
            res.n_processed += len(prompt) - m
            admitted.append((req, prompt, m, node, row))
        if leaf:
            for _ in range(cfg.decode_steps):
                new = cache.alloc(len(admitted))
                for (_, _, _, _, row), s in zip(admitted, new):
                    row.append(s)
        for req, prompt, m, node, row in admitted:
            seq = np.concatenate([prompt, wl.decode_tokens(req)]) if req.decode_steps else prompt
            k, _ = cache.insert(seq, row)
            cache.free(row[m:k])
            cache.unlock(node)
            res.present[req.rid] = k
            res.rows[req.rid] = np.asarray(row, np.int32)
        for req, _, m, _, _ in admitted:
            if want is not None and req.rid not in want:
                continue
            if m != req.prompt_len - req.own_len:
                raise RuntimeError(f"request {req.rid}: matched {m}, synthetic queries "
                                   f"cover only the last {req.own_len} tokens")
            res.extend_out[req.rid], res.decode_out[req.rid] = request_attention(wl, req)
    leaves = wl.leaf_requests
    res.n_logical = sum(r.prompt_len for r in leaves)
    res.r_saving = r_saving(res.n_processed, res.n_logical)
    res.hit_rate = hit_rate(sum(res.matched[r.rid] for r in leaves), res.n_logical)
    res.stats = cache.stats()
    return res

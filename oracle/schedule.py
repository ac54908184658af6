"""Cache-aware request ordering (oracle; test infrastructure only: tests,
the smoke check and the benchmark's CPU leg import it, never the product).

Passages followed:
  * SGLang paper notes (section 3, cache-aware scheduling; appendix A.2, the
    scheduling pseudocode; appendix A.3, the proof of Theorem 3.1): the cache
    hit rate is the number of cached prompt tokens over the number of prompt
    tokens; the waiting requests are matched against the radix tree and run
    longest shared prefix first instead of in arrival order; that order is a
    depth-first order of the batch's radix tree and, when the cache holds at
    least the longest request, computes the KV of every edge of that tree
    exactly once, so the hit rate reaches 1 - C / (prompt tokens), C the total
    edge length -- the optimum.
  * vLLM-vs-SGLang page, cache-aware ordering: SGLang's longest-prefix-match
    policy is optional (arrival order is the default) and goes back to arrival
    order when more than 128 requests wait.

Readings of points the pages leave open (the product's scheduler follows the
same):
  * the longest-shared-prefix-first order is built greedily within one
    scheduling round: the next request is the one whose prompt shares the
    longest prefix with the cache or with a request already placed in the
    round (its tokens will be cached by the time the later request runs);
    ties go to the earliest arrival;
  * the shared lengths are counted in whole matching units (rounded down),
    as an admission counts its match;
  * matching for ordering leaves the cache as it is (no split, no LRU stamp);
  * more than `fcfs_above` (128) waiting requests: arrival order, no matching.
"""
from __future__ import annotations

from .cache_model import TokenTrieCache


def lcp(a, b) -> int:
    """Length of the longest common prefix of two token sequences."""
    n = min(len(a), len(b))
    i = 0
    while i < n and int(a[i]) == int(b[i]):
        i += 1
    return i


def peek_match(cache: TokenTrieCache, tokens) -> int:
    """Matched length of `tokens` against the cache, rounded down to the
    matching unit, without touching the cache (no split, no clock tick)."""
    cur, n = cache.root, 0
    for t in tokens:
        nxt = cur.children.get(int(t))
        if nxt is None:
            break
        n += 1
        cur = nxt
    return (n // cache.unit) * cache.unit


def lpm_order(cache: TokenTrieCache, prompts, fcfs_above: int = 128):
    """Longest-shared-prefix-first order of the waiting `prompts` (listed in
    arrival order) -> (order, score of each placed request when placed)."""
    n = len(prompts)
    if n > fcfs_above:
        return list(range(n)), [0] * n
    unit = cache.unit
    best = [peek_match(cache, p) for p in prompts]
    placed = [False] * n
    order, scores = [], []
    for _ in range(n):
        pick = -1
        for i in range(n):
            if not placed[i] and (pick < 0 or best[i] > best[pick]):
                pick = i
        placed[pick] = True
        order.append(pick)
        scores.append(best[pick])
        for j in range(n):
            if not placed[j]:
                s = (lcp(prompts[j], prompts[pick]) // unit) * unit
                best[j] = max(best[j], s)
    return order, scores


def dfs_order(prompts):
    """A depth-first order of the batch's token trie: at every trie node the
    requests ending there come first (by arrival), then the child subtrees in
    the order of the earliest arrival inside each."""
    root = {"end": [], "kids": {}, "first": None}
    for i, p in enumerate(prompts):
        node = root
        if node["first"] is None:
            node["first"] = i
        for t in p:
            node = node["kids"].setdefault(int(t), {"end": [], "kids": {}, "first": None})
            if node["first"] is None:
                node["first"] = i
        node["end"].append(i)
    out = []

    def visit(node):
        out.extend(node["end"])
        for kid in sorted(node["kids"].values(), key=lambda k: k["first"]):
            visit(kid)

    visit(root)
    return out


def batch_tree_tokens(prompts) -> int:
    """C: the number of distinct prefixes of the batch (total edge length of its
    radix tree), i.e. tokens whose KV must be computed at least once."""
    seen = set()
    for p in prompts:
        for k in range(1, len(p) + 1):
            seen.add(tuple(int(t) for t in p[:k]))
    return len(seen)


def run_order(prompts, order, capacity: int, match_unit: int = 1, cache: TokenTrieCache | None = None):
    """Runs the requests one after another in `order` on a cache of `capacity`
    slots (each request: match, lock, allocate its uncached suffix, insert its
    prompt, free its duplicates, unlock) -> (cached prompt tokens, prompt
    tokens).  The hit rate is their ratio."""
    c = cache if cache is not None else TokenTrieCache(capacity, match_unit)
    cached = total = 0
    for i in order:
        p = [int(t) for t in prompts[i]]
        m, slots, node = c.match_prefix(p)
        if node:
            c.lock(node)
        new = c.alloc(len(p) - m)
        k, _ = c.insert(p, list(slots) + list(new))
        c.free(new[: k - m])
        if node:
            c.unlock(node)
        cached += m
        total += len(p)
    return cached, total

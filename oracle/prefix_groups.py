"""Global prefix analysis (oracle; test infrastructure only: tests, the smoke
check and the benchmark's CPU leg import it, never the product).

Passage followed: BatchLLM explainer, Global Prefix Sharing.  All requests
of a batch are inserted into one radix tree; requests that share a prefix
are scheduled as a group whose common prefix is computed once, and each
member computes the rest of its prompt on its own (a group is one shared
level, as the explainer's two-part attention assumes).  A dynamic program
over the tree decides, node by node, whether the leaves below keep one group
here or are split into groups further down; the explainer states the local
test: a grandchild c' is worth its own group when gain(c') =
(leaves(c') - 1) x tokens(c') exceeds the penalty tokens(c) of recomputing
the child's tokens for it.  The token saving is R_saving = 1 -
N_processed / N_logical (Equation 2).

What is computed here is the plain definition the program reaches: over
every way to give each request a group node on its path (the group's prefix
= the tokens from the root to that node), the least

    N_processed = sum over groups of their prefix length
                + sum over requests of (prompt length - its group's prefix)

and a grouping that reaches it.  Readings: a request whose prompt ends at a
node may be grouped there (its whole prompt is then the prefix); on ties a
node keeps one group for everything below (fewer, larger groups); groups
are numbered in order of their first request.
"""
from __future__ import annotations


def _trie(prompts):
    root = {"kids": {}, "reqs": [], "depth": 0}
    for i, p in enumerate(prompts):
        node = root
        node["reqs"].append(i)
        for d, t in enumerate(p, 1):
            node = node["kids"].setdefault(int(t), {"kids": {}, "reqs": [], "depth": d})
            node["reqs"].append(i)
    return root


def min_processed(prompts):
    """-> (N_processed, group id per request, prefix length per request)."""
    lens = [len(p) for p in prompts]
    root = _trie(prompts)
    # children before parents (explicit stack: prompts can be long)
    order, stack = [], [root]
    while stack:
        node = stack.pop()
        order.append(node)
        stack.extend(node["kids"].values())
    cost, here_wins = {}, {}
    for node in reversed(order):
        d = node["depth"]
        # every request below is grouped here ...
        here = d + sum(lens[r] - d for r in node["reqs"])
        if not node["kids"]:
            cost[id(node)], here_wins[id(node)] = here, True
            continue
        # ... or the requests ending here form a group here and each child
        # subtree is grouped on its own
        ending = any(lens[r] == d for r in node["reqs"])
        split = (d if ending else 0) + sum(cost[id(k)] for k in node["kids"].values())
        here_wins[id(node)] = here <= split
        cost[id(node)] = min(here, split)
    group_node = [None] * len(prompts)
    stack = [root]
    while stack:
        node = stack.pop()
        if here_wins[id(node)]:
            for r in node["reqs"]:
                group_node[r] = node
            continue
        for r in node["reqs"]:
            if lens[r] == node["depth"]:
                group_node[r] = node
        stack.extend(node["kids"].values())
    ids, group, prefix = {}, [], []
    for r in range(len(prompts)):
        g = group_node[r]
        ids.setdefault(id(g), len(ids))
        group.append(ids[id(g)])
        prefix.append(g["depth"])
    return cost[id(root)], group, prefix


def processed_of(prompts, group, prefix) -> int:
    """N_processed of a given grouping (each group's prefix once, the rest of
    every prompt per request)."""
    seen = {}
    for g, p in zip(group, prefix):
        seen[g] = p
    return sum(seen.values()) + sum(len(q) - p for q, p in zip(prompts, prefix))


def r_saving(n_processed: int, n_logical: int) -> float:
    """Equation 2, in percent."""
    return (1.0 - n_processed / n_logical) * 100.0

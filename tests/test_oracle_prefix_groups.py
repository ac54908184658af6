"""Pins of the oracle's global prefix analysis (oracle/prefix_groups.py):
brute force over every grouping of small batches, the explainer's local
gain-versus-penalty test, the token savings the BatchLLM explainer prints
(golden token_saving.json) and the closed forms of the workload shapes."""
import itertools
import json
import os

import numpy as np
import pytest

from oracle.prefix_groups import min_processed, processed_of, r_saving

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "token_saving.json")


def _brute(prompts):
    """Least N_processed over every assignment of a group node (a prefix
    length of the request's own prompt) to each request; requests in one
    group share the same node, i.e. the same prefix tokens."""
    best = None
    for cut in itertools.product(*[range(len(p) + 1) for p in prompts]):
        nodes = {tuple(p[:c]) for p, c in zip(prompts, cut)}
        n = sum(len(x) for x in nodes) + sum(len(p) - c for p, c in zip(prompts, cut))
        best = n if best is None else min(best, n)
    return best


@pytest.mark.parametrize("seed", range(40))
def test_brute_force_optimum(seed):
    rng = np.random.default_rng(seed)
    n = 2 + seed % 4
    prompts = [[int(x) for x in rng.integers(0, 2, int(rng.integers(0, 5)))] for _ in range(n)]
    total, group, prefix = min_processed(prompts)
    assert total == _brute(prompts)
    # the grouping reaches it, and every group's members share its prefix
    assert processed_of(prompts, group, prefix) == total
    for g in set(group):
        mem = [i for i in range(n) if group[i] == g]
        assert len({prefix[i] for i in mem}) == 1
        assert len({tuple(prompts[i][: prefix[i]]) for i in mem}) == 1


def _two_level(t_c, t1, n1, t2, n2):
    """root -> c (t_c tokens) -> c'1 (t1 tokens, n1 requests of one own token
    each) and c'2 (t2 tokens, n2 requests)."""
    c = [1] * t_c
    a = [c + [2] + [3] * (t1 - 1) + [10 + i] for i in range(n1)]
    b = [c + [4] + [5] * (t2 - 1) + [20 + i] for i in range(n2)]
    return a + b


@pytest.mark.parametrize("t_c,t1,n1,split", [(10, 4, 4, True), (12, 4, 4, False), (11, 4, 4, True),
                                             (30, 4, 4, False), (3, 2, 3, True), (4, 2, 3, False)])
def test_gain_versus_penalty(t_c, t1, n1, split):
    """c'1 gets a group of its own exactly when (leaves - 1) x tokens of c'1
    exceeds the tokens of c (ties stay merged); c'2's lone request computes
    its whole prompt either way."""
    prompts = _two_level(t_c, t1, n1, 3, 1)
    assert ((n1 - 1) * t1 > t_c) == split
    total, group, prefix = min_processed(prompts)
    assert len(set(group[:n1])) == 1
    lone = t_c + 3 + 1
    if split:
        assert prefix[0] == t_c + t1 and group[0] != group[n1]
        assert total == (t_c + t1) + n1 + lone
    else:
        assert prefix[0] == t_c and group[0] == group[n1]
        assert total == t_c + n1 * (t1 + 1) + (lone - t_c)


def _shape(levels, seed=0):
    """Prompts of a sharing tree: levels = ((fanout, length), ...)."""
    rng = np.random.default_rng(seed)
    nxt = [0]

    def fresh(n):
        nxt[0] += n
        return list(range(nxt[0] - n, nxt[0]))   # distinct tokens: an exact tree

    paths = [[]]
    for fan, length in levels:
        paths = [p + fresh(length) for p in paths for _ in range(fan)]
    return paths


def test_printed_savings():
    """BatchLLM explainer, token-saving section: prefix 2,000 shared by 16 with
    200 distinct tokens saves 85.2 %; prefix 16,000 saves 92.6 %."""
    gold = json.load(open(GOLDEN))
    for prefix_len in (2000, 16000):
        prompts = _shape(((1, prefix_len), (16, 200)))
        total, group, prefix = min_processed(prompts)
        assert total == prefix_len + 16 * 200 and len(set(group)) == 1
        printed = [e["percent"] for e in gold["r_saving_printed"] if e["prefix"] == prefix_len][0]
        got = r_saving(total, sum(len(p) for p in prompts))
        assert abs(got - printed) <= gold["r_saving_printed_precision"]


def test_multilevel_groups_at_the_branches():
    """Root 1,024 -> 8 branches of 512 -> 3 forks of 128 (scaled by 1/8 here):
    one group at the root recomputes every branch per fork, groups at the
    forks recompute the root and branch per fork; groups at the branches
    compute the root once per branch and win."""
    prompts = _shape(((1, 128), (8, 64), (3, 16)))
    total, group, prefix = min_processed(prompts)
    assert total == 8 * (128 + 64) + 24 * 16
    assert len(set(group)) == 8 and set(prefix) == {192}
    assert total < 128 + 24 * (64 + 16) and total < 24 * (128 + 64 + 16)

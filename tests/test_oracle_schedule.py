"""Pins of the oracle's cache-aware ordering (oracle/schedule.py).

Theorem 3.1 of the SGLang paper (notes: appendix A.3): when the cache holds at
least the longest request, running a batch in a depth-first order of its
radix tree computes every edge's KV exactly once, so the cached prompt tokens
reach (prompt tokens - C), C the tree's total edge length, and no order does
better (every distinct prefix is computed at least once).  The brute force
below runs every order of small random batches through the cache model and
checks that maximum, that the depth-first order reaches it and that the
longest-shared-prefix-first order reaches it too (the paper calls the two
orders equivalent)."""
import itertools

import numpy as np
import pytest

from oracle import schedule as sch
from oracle.cache_model import TokenTrieCache


def _random_batch(rng, n):
    # small alphabet and short prompts: plenty of shared prefixes, some duplicates
    return [list(rng.integers(0, 3, size=int(rng.integers(1, 7)))) for _ in range(n)]


@pytest.mark.parametrize("seed", range(40))
def test_brute_force_optimum_is_reached_by_dfs_and_lpm_orders(seed):
    rng = np.random.default_rng(seed)
    n = 3 + seed % 3  # 3..5 requests (up to 120 orders)
    prompts = _random_batch(rng, n)
    longest = max(len(p) for p in prompts)
    total = sum(len(p) for p in prompts)
    c_edges = sch.batch_tree_tokens(prompts)
    for capacity in (longest, longest + int(rng.integers(0, 4))):
        best = max(sch.run_order(prompts, perm, capacity)[0] for perm in itertools.permutations(range(n)))
        assert best == total - c_edges
        assert sch.run_order(prompts, sch.dfs_order(prompts), capacity)[0] == best
        order, _ = sch.lpm_order(TokenTrieCache(capacity), prompts)
        assert sorted(order) == list(range(n))
        assert sch.run_order(prompts, order, capacity)[0] == best


def test_six_requests_brute_force():
    rng = np.random.default_rng(1234)
    for _ in range(3):
        prompts = _random_batch(rng, 6)
        capacity = max(len(p) for p in prompts)
        best = max(sch.run_order(prompts, perm, capacity)[0] for perm in itertools.permutations(range(6)))
        assert best == sum(len(p) for p in prompts) - sch.batch_tree_tokens(prompts)
        order, _ = sch.lpm_order(TokenTrieCache(capacity), prompts)
        assert sch.run_order(prompts, order, capacity)[0] == best


def test_arrival_order_can_lose_what_lpm_keeps():
    """A prompt sharing a prefix with an earlier one, separated by an unrelated
    prompt: in arrival order the shared prefix is evicted before it is reused
    (a cache just big enough for the longest request); placing the related
    prompts together keeps it.  Also fails if the ordering forgot to count the
    requests already placed in the round (all scores would stay 0)."""
    a, x, b = [0, 1, 2], [5], [0, 1, 3]
    prompts = [a, x, b]
    assert sch.run_order(prompts, [0, 1, 2], 3)[0] == 0
    order, scores = sch.lpm_order(TokenTrieCache(3), prompts)
    assert order == [0, 2, 1] and scores == [0, 2, 0]
    assert sch.run_order(prompts, order, 3)[0] == 2


def test_ties_go_to_the_earliest_arrival_and_cached_prefixes_first():
    cache = TokenTrieCache(64)
    sch.run_order([[7, 7, 7, 7]], [0], 64, cache=cache)  # cache holds 7 7 7 7
    prompts = [[1, 2], [7, 7, 9], [3], [7, 7, 7, 7, 1], [1, 5]]
    order, scores = sch.lpm_order(cache, prompts)
    # 3 has the longest cached prefix (4), then 1 (shares 2 with the cache);
    # then 0 and 2 and 4 tie at 0 -> arrival order, except that 4 shares 1 with 0
    assert order == [3, 1, 0, 4, 2]
    assert scores == [4, 2, 0, 1, 0]


def test_matching_unit_counts_whole_units():
    cache = TokenTrieCache(64, match_unit=2)
    sch.run_order([[4, 4, 4]], [0], 64, cache=cache)
    assert sch.peek_match(cache, [4, 4, 4, 1]) == 2
    order, scores = sch.lpm_order(cache, [[9], [4, 4, 4, 1], [9, 9]])
    assert order == [1, 0, 2] and scores == [2, 0, 0]


def test_fcfs_above_the_queue_limit_and_peek_has_no_side_effects():
    cache = TokenTrieCache(64)
    sch.run_order([[1, 2, 3]], [0], 64, cache=cache)
    before = (cache.clock, cache.next_id, len(cache.segs))
    assert sch.peek_match(cache, [1, 2, 9]) == 2
    assert (cache.clock, cache.next_id, len(cache.segs)) == before
    prompts = [[0]] * 3 + [[1, 2, 3]]
    assert sch.lpm_order(cache, prompts, fcfs_above=3)[0] == [0, 1, 2, 3]
    assert sch.lpm_order(cache, prompts, fcfs_above=4)[0] == [3, 0, 1, 2]


def test_dfs_order_groups_subtrees():
    prompts = [[0, 1, 2], [5], [0, 1, 3], [0, 4], [5, 6]]
    assert sch.dfs_order(prompts) == [0, 2, 3, 1, 4]
    assert sch.batch_tree_tokens(prompts) == 7

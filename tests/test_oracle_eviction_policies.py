"""Pins of the oracle's eviction policies (LRU, LFU, SLRU, priority).

Hand-worked histories where the policies disagree on the victim, the
textbook order each one stands for, the bookkeeping across splits, and a
property every policy keeps: the victim is always an unreferenced leaf."""
import numpy as np
import pytest

from oracle.cache_model import POLICIES, CacheError, TokenTrieCache


def _serve(c, seq):
    """One request: match, lock, allocate the rest, insert, free, unlock."""
    m, slots, node = c.match_prefix(seq)
    if node:
        c.lock(node)
    new = c.alloc(len(seq) - m)
    k, _ = c.insert(seq, list(slots) + new)
    c.free(new[: k - m])
    if node:
        c.unlock(node)


def _resident(c):
    return sorted(tuple(s) for s in c.resident_sequences())


A, B, C = [1, 2, 3], [4, 5, 6], [7, 8, 9]


def _history(policy, prio_a=0, prio_b=0):
    """A served (its insert creates it: 1 access), then re-read twice (3
    accesses, last at clock 4); B served after (1 access, clock 6).  The pool
    holds both; C then needs 3 slots: one of A, B goes."""
    c = TokenTrieCache(6, policy=policy)
    c.set_priority(prio_a)
    _serve(c, A)
    c.match_prefix(A)
    c.match_prefix(A)
    c.set_priority(prio_b)
    _serve(c, B)
    c.set_priority(0)
    _serve(c, C)
    return _resident(c)


def test_lru_evicts_the_least_recently_used():
    assert _history("lru") == [tuple(B), tuple(C)]


def test_lfu_evicts_the_least_frequently_used():
    # A: insert + 2 matches = 3 accesses (its first match hit nothing); B: 1
    assert _history("lfu") == [tuple(A), tuple(C)]


def test_slru_evicts_probation_before_protected():
    # A was re-read (protected), B only inserted (probation)
    assert _history("slru") == [tuple(A), tuple(C)]


def test_priority_evicts_the_lowest_priority():
    assert _history("priority", prio_a=1, prio_b=0) == [tuple(A), tuple(C)]
    # equal priorities fall back to LRU
    assert _history("priority") == [tuple(B), tuple(C)]
    # and a high-priority B is kept
    assert _history("priority", prio_a=0, prio_b=2) == [tuple(B), tuple(C)]


def test_lfu_and_slru_differ():
    """A accessed 3 times long ago, B twice recently: LFU takes B (fewer
    accesses), SLRU takes A (both protected, A older)."""
    out = {}
    for pol in ("lfu", "slru"):
        c = TokenTrieCache(6, policy=pol)
        _serve(c, A)
        c.match_prefix(A)
        c.match_prefix(A)       # A: 3 accesses
        _serve(c, B)
        c.match_prefix(B)       # B: 2 accesses, more recent
        _serve(c, C)
        out[pol] = _resident(c)
    assert out["lfu"] == [tuple(A), tuple(C)]
    assert out["slru"] == [tuple(B), tuple(C)]


def test_split_copies_accesses_and_priority():
    c = TokenTrieCache(16, policy="lfu")
    c.set_priority(3)
    _serve(c, [1, 2, 3, 4])
    c.set_priority(1)
    m, _, node = c.match_prefix([1, 2, 9])   # splits [1,2] | [3,4]
    assert m == 2
    up = c.node_info(node)
    low = [c.node_info(s) for s in c.segs if s != node][0]
    # the upper part: the old counters, then this call's access
    assert (up["hits"], up["prio"]) == (2, 3)
    assert (low["hits"], low["prio"]) == (1, 3)
    c.set_priority(7)
    c.match_prefix([1, 2])
    assert (c.node_info(node)["hits"], c.node_info(node)["prio"]) == (3, 7)


@pytest.mark.parametrize("policy", POLICIES)
def test_victims_are_unreferenced_leaves(policy):
    rng = np.random.default_rng(len(policy))
    c = TokenTrieCache(40, policy=policy)
    held = []
    for step in range(200):
        c.set_priority(int(rng.integers(0, 3)))
        seq = [int(x) for x in rng.integers(0, 3, int(rng.integers(1, 8)))]
        m, slots, node = c.match_prefix(seq)
        if node:
            c.lock(node)
        pinned_before = {s.id for s in c.segs.values() if s.ref > 0}
        try:
            new = c.alloc(len(seq) - m)
        except CacheError:
            if node:
                c.unlock(node)
            continue
        assert pinned_before <= set(c.segs)   # alloc evicted nothing referenced
        k, _ = c.insert(seq, list(slots) + new)
        c.free(new[: k - m])
        held.append(node)
        if len(held) > 3:
            n = held.pop(0)
            if n:
                c.unlock(n)


def test_unknown_policy():
    with pytest.raises(CacheError):
        TokenTrieCache(8, policy="fifo")

"""Pins of the oracle's cache model.

Checked against: the pages' worked prefix-match example (golden fixture),
the matching-unit loss bound, a brute-force definition of the match length
(longest common prefix with any resident sequence), the SGLang Figure 3
eviction narrative, and an LRU property tracked per token independently of
the model's segment bookkeeping.
"""
import json
import os

import numpy as np
import pytest

from oracle import CacheError, ENOSPC, ESTATE, TokenTrieCache

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _serve(cache, prompt, gen=()):
    """match, lock, allocate, insert prompt+gen, free duplicates, unlock."""
    m, slots, node = cache.match_prefix(prompt)
    cache.lock(node)
    seq = list(prompt) + list(gen)
    row = list(slots) + cache.alloc(len(seq) - m)
    k, _ = cache.insert(seq, row)
    cache.free(row[m:k])
    cache.unlock(node)
    return m


@pytest.mark.parametrize("unit_key,unit", [("saved_unit1", 1), ("saved_unit16", 16)])
def test_worked_example_saved_tokens(unit_key, unit):
    gold = json.load(open(os.path.join(GOLD, "worked_example_prefix_match.json")))
    rng = np.random.default_rng(3)
    common = list(rng.choice(np.arange(1000, 30000), gold["common_prefix_tokens"], replace=False))
    for case in gold["cases"]:
        cache = TokenTrieCache(10_000, unit)
        saved = []
        for i in range(3):                        # first request fills the cache
            parts = {"common": common,
                     "timestamp": [100 + i],
                     "question": [40000 + 100 * i + j for j in range(gold["question_tokens"])]}
            prompt = [t for name in case["layout"] for t in parts[name]]
            answer = [50000 + 10000 * i + j for j in range(case["answer_tokens"])]
            saved.append(_serve(cache, prompt, answer))
        assert saved[0] == 0
        assert saved[1:] == [case[unit_key]] * 2, case["case"]


def test_matching_unit_loss_bound():
    gold = json.load(open(os.path.join(GOLD, "worked_example_prefix_match.json")))
    bound = gold["max_loss_per_request_unit16"]
    rng = np.random.default_rng(4)
    c1, c16 = TokenTrieCache(50_000, 1), TokenTrieCache(50_000, 16)
    base = list(rng.integers(0, 50, 300))
    seen = set()
    for _ in range(60):
        cut = int(rng.integers(0, 300))
        prompt = base[:cut] + list(rng.integers(0, 50, int(rng.integers(1, 40))))
        m1, m16 = _serve(c1, prompt), _serve(c16, prompt)
        assert m16 % 16 == 0
        assert 0 <= m1 - m16 <= bound
        seen.add(m1 - m16)
    assert max(seen) > 8          # the bound is actually approached


def _lcp(a, b):
    n = 0
    for x, y in zip(a, b):
        if x != y:
            break
        n += 1
    return n


def test_match_length_is_longest_common_prefix_with_resident_sequences():
    rng = np.random.default_rng(5)
    for trial in range(20):
        cache = TokenTrieCache(200)
        for _ in range(25):
            seq = list(rng.integers(0, 3, int(rng.integers(1, 10))))
            resident = cache.resident_sequences()
            brute = max([_lcp(seq, r) for r in resident], default=0)
            m, slots, node = cache.match_prefix(seq)
            assert m == brute
            assert len(slots) == m
            cache.lock(node)
            try:
                row = list(slots) + cache.alloc(len(seq) - m)
            except CacheError as e:
                assert e.code == ENOSPC
                cache.unlock(node)
                continue
            k, _ = cache.insert(seq, row)
            cache.free(row[m:k])
            cache.unlock(node)
            free, tree, priv = cache.slot_partition()
            assert not priv and len(free) + len(tree) == 200 and not (free & tree)


def test_figure3_eviction_narrative():
    """SGLang paper notes, Figure 3: a chat session inserted (2), extended
    (3); a second session splits the shared system prompt (4); under memory
    pressure the stale turn of session 1 is evicted (5); a few-shot query
    with no shared prefix hangs off the root (6); more queries split the
    few-shot node (7); session 1 returns and session 2's nodes go (8);
    sampling more answers for one query evicts three other query leaves (9).
    Lengths and the capacity are chosen to force exactly these evictions."""
    SYS, U1A1, U2A2, U3A3, U4A4, U5A5 = [1, 2], [3, 4], list(range(10, 20)), [5, 6], [7, 8], [21, 22, 23, 24, 25, 26, 27]
    FS, Q = [30], {i: [40 + i] for i in range(1, 5)}
    cache = TokenTrieCache(17)

    def resident_prefixes():
        return {tuple(s) for s in cache.resident_sequences()}

    _serve(cache, SYS + U1A1)                                      # (2)
    _serve(cache, SYS + U1A1, U2A2)                                # (3)
    assert cache.stats()["nodes"] == 2
    _serve(cache, SYS, U3A3)                                       # (4) split of the shared prompt
    assert cache.stats()["nodes"] == 4
    ev = cache.stats()["evictions"]
    _serve(cache, SYS + U3A3, U4A4)                                # (5)
    assert cache.stats()["evictions"] == ev + 1
    assert tuple(SYS + U1A1 + U2A2) not in resident_prefixes()
    assert tuple(SYS + U1A1) in resident_prefixes()
    _serve(cache, FS + Q[1])                                       # (6)
    for i in (2, 3, 4):                                            # (7)
        _serve(cache, FS + Q[i])
    assert cache.stats()["evictions"] == ev + 1
    _serve(cache, SYS + U1A1, U5A5)                                # (8)
    res = resident_prefixes()
    assert cache.stats()["evictions"] == ev + 3
    assert not any(s[:3] == tuple(SYS + U3A3[:1]) for s in res)    # session 2 gone
    assert tuple(SYS + U1A1 + U5A5) in res
    _serve(cache, FS + Q[2], [90, 91, 92, 93])                     # (9)
    res = resident_prefixes()
    assert cache.stats()["evictions"] == ev + 6
    for i in (1, 3, 4):
        assert tuple(FS + Q[i]) not in res
    assert tuple(FS + Q[2] + [90, 91, 92, 93]) in res
    assert tuple(SYS + U1A1 + U5A5) in res


def test_lru_property_tracked_per_token():
    """Track each resident token's last walk time independently (a walk
    covering a prefix refreshes every token of it).  Whenever tokens are
    evicted, none may have been walked after any surviving unlocked token,
    and no locked token may go."""
    rng = np.random.default_rng(6)
    for trial in range(30):
        cache = TokenTrieCache(24)
        t_walk = {}              # prefix tuple -> last walk tick
        tick = 0
        active = []              # (prompt, m, node, row)
        for _ in range(60):
            before = {p for s in cache.resident_sequences() for p in (tuple(s[:i]) for i in range(1, len(s) + 1))}
            locked = {tuple(pr[:i]) for pr, m, _, _ in active for i in range(1, m + 1)}
            op = rng.random()
            if op < 0.5 or not active:
                seq = list(rng.integers(0, 3, int(rng.integers(1, 8))))
                m, slots, node = cache.match_prefix(seq)
                tick += 1
                for i in range(1, m + 1):
                    t_walk[tuple(seq[:i])] = tick
                cache.lock(node)
                try:
                    row = list(slots) + cache.alloc(len(seq) - m)
                    active.append((seq, m, node, row))
                except CacheError as e:
                    assert e.code == ENOSPC
                    cache.unlock(node)
            elif op < 0.85:
                seq, m, node, row = active.pop(int(rng.integers(0, len(active))))
                k, _ = cache.insert(seq, row)
                tick += 1
                for i in range(1, len(seq) + 1):
                    t_walk[tuple(seq[:i])] = tick
                cache.free(row[m:k])
                cache.unlock(node)
            else:
                cache.evict(int(rng.integers(1, 6)))
            after = {p for s in cache.resident_sequences() for p in (tuple(s[:i]) for i in range(1, len(s) + 1))}
            gone = before - after
            if gone:
                assert not (gone & locked)
                survivors = [t_walk[p] for p in after if p not in locked and p in before]
                if survivors:
                    assert max(t_walk[p] for p in gone) <= min(survivors)


def test_error_paths_leave_state_unchanged():
    cache = TokenTrieCache(8)
    m, slots, node = cache.match_prefix([1, 2, 3])
    cache.lock(node)
    row = cache.alloc(3)
    k, leaf = cache.insert([1, 2, 3], row)
    cache.lock(leaf)
    snap = cache.stats()
    with pytest.raises(CacheError) as e:
        cache.alloc(6)                    # 5 free, nothing evictable (locked)
    assert e.value.code == ENOSPC and cache.stats() == snap
    with pytest.raises(CacheError) as e:
        cache.free([row[0]])              # a tree slot, not a private one
    assert e.value.code == ESTATE and cache.stats() == snap
    cache.unlock(leaf)
    with pytest.raises(CacheError) as e:
        cache.unlock(leaf)                # underflow
    assert e.value.code == ESTATE
    priv = cache.alloc(2)
    cache.free(priv)
    with pytest.raises(CacheError) as e:
        cache.free(priv)                  # double free
    assert e.value.code == ESTATE

"""The C++ radix tree (edge-compressed) against the oracle's token-level
trie: random sequences of match / lock / alloc / insert / free / unlock /
evict, with pools small enough to force eviction; every returned length,
slot list, node id, freed count, error code and statistic must be equal."""
import numpy as np
import pytest

from oracle import CacheError, TokenTrieCache
from prefix_shared_kv_token_amd import rdx


def _call(fn, *a):
    try:
        return ("ok", fn(*a))
    except rdx.RdxError as e:
        return ("err", e.code)
    except CacheError as e:
        return ("err", e.code)


def _norm(x):
    if isinstance(x, tuple):
        return tuple(_norm(v) for v in x)
    if isinstance(x, np.ndarray):
        return [int(v) for v in x]
    if isinstance(x, list):
        return [int(v) for v in x]
    return x


def _same(a, b):
    assert _norm(a) == _norm(b), (a, b)


def _stats_eq(tree, model):
    s, o = tree.stats(), model.stats()
    assert s == o, (s, o)


def _run(seed, num_slots, unit, vocab, max_len, steps, policy="lru"):
    rng = np.random.default_rng(seed)
    tree, model = rdx.Tree(num_slots, unit, policy), TokenTrieCache(num_slots, unit, policy)
    active = []
    for step in range(steps):
        op = rng.random()
        if policy == "priority" and rng.random() < 0.3:
            p = int(rng.integers(0, 4))
            tree.set_priority(p)
            model.set_priority(p)
        if op < 0.4 or not active:
            seq = list(rng.integers(0, vocab, int(rng.integers(0, max_len))))
            a = _call(tree.match_prefix, seq)
            b = _call(model.match_prefix, seq)
            _same(a, b)
            m, slots, node = b[1]
            _same(_call(tree.lock, node), _call(model.lock, node))
            extra = int(rng.integers(0, 4))
            gen = list(rng.integers(0, vocab, extra))
            a = _call(tree.alloc, len(seq) + extra - m)
            b = _call(model.alloc, len(seq) + extra - m)
            _same(a, b)
            if b[0] == "ok":
                active.append((seq + gen, m, node, list(slots) + list(b[1])))
            else:
                _same(_call(tree.unlock, node), _call(model.unlock, node))
        elif op < 0.75:
            seq, m, node, row = active.pop(int(rng.integers(0, len(active))))
            a, b = _call(tree.insert, seq, row), _call(model.insert, seq, row)
            _same(a, b)
            if b[0] == "err":      # a random unlock below released this request's lock
                continue
            k = b[1][0]
            _same(_call(tree.free, row[m:k]), _call(model.free, row[m:k]))
            _same(_call(tree.unlock, node), _call(model.unlock, node))
        elif op < 0.85:
            n = int(rng.integers(0, 8))
            _same(_call(tree.evict, n), _call(model.evict, n))
        elif op < 0.92:
            # illegal or unusual calls must fail (or succeed) the same way
            nid = int(rng.integers(0, model.next_id + 2))
            _same(_call(tree.unlock, nid), _call(model.unlock, nid))
            s = int(rng.integers(0, num_slots))
            _same(_call(tree.free, [s]), _call(model.free, [s]))
        else:
            for nid in list(model.segs)[:5]:
                info, ref = tree.node(nid), model.node_info(nid)
                assert (info["start"], info["length"], info["ref"], info["last_access"], info["hits"],
                        info["priority"]) == (ref["start"], ref["length"], ref["ref"], ref["last"], ref["hits"],
                                              ref["prio"])
                assert list(info["slots"]) == ref["slots"]
        _stats_eq(tree, model)
    return model


@pytest.mark.parametrize("seed", range(40))
def test_random_ops_unit1(seed):
    model = _run(seed, num_slots=30, unit=1, vocab=3, max_len=9, steps=120)
    assert model.evictions > 0 or seed % 7 == 0


@pytest.mark.parametrize("seed", range(10))
def test_random_ops_unit16(seed):
    _run(100 + seed, num_slots=400, unit=16, vocab=2, max_len=60, steps=80)


@pytest.mark.parametrize("seed", range(5))
def test_random_ops_large_vocab(seed):
    _run(200 + seed, num_slots=200, unit=1, vocab=50, max_len=30, steps=150)


@pytest.mark.parametrize("policy", ["lfu", "slru", "priority"])
@pytest.mark.parametrize("seed", range(12))
def test_random_ops_eviction_policies(seed, policy):
    model = _run(300 + seed, num_slots=30, unit=1 + (seed % 3 == 2), vocab=3, max_len=9, steps=150, policy=policy)
    assert model.evictions > 0 or seed % 5 == 0


def test_reuse_stream_hit_rates_equal_the_oracle():
    """The measured eviction stream (400 requests, pool of 6,000 slots):
    the cached prompt tokens under every policy equal the oracle's."""
    from workloads import reuse_stream

    prompts, hot = reuse_stream()

    def serve(c, prio):
        cached = 0
        for p, h in zip(prompts, hot):
            if prio:
                c.set_priority(int(h))
            m, slots, node = c.match_prefix(p)
            if node:
                c.lock(node)
            new = c.alloc(len(p) - m)
            k, _ = c.insert(p, list(slots) + list(new))
            if k > m:
                c.free(list(new)[: k - m])
            if node:
                c.unlock(node)
            cached += m
        return cached

    for pol in ("lru", "lfu", "slru", "priority"):
        prio = pol == "priority"
        assert serve(rdx.Tree(6000, 1, pol), prio) == serve(TokenTrieCache(6000, 1, pol), prio), pol

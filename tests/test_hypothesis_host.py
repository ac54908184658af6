"""Property-based (hypothesis) cross-checks of the host algorithms against
the oracle: the C++ radix tree under arbitrary operation sequences (small
pools, so allocations evict), the token batcher on arbitrary jobs, the global
prefix analysis and the cache-aware order on arbitrary batches.  Every
result must equal the oracle's bit for bit; hypothesis shrinks any failure to
a minimal case."""
import numpy as np
from hypothesis import HealthCheck, given, settings, strategies as st

from oracle import CacheError, TokenTrieCache
from oracle import schedule as osch
from oracle.prefix_groups import min_processed
from oracle.token_batching import Group, batch_iterations
from prefix_shared_kv_token_amd import rdx

SETTINGS = settings(max_examples=120, deadline=None, suppress_health_check=[HealthCheck.too_slow])

seqs = st.lists(st.integers(0, 2), min_size=0, max_size=8)
ops = st.lists(st.tuples(st.sampled_from(["serve", "hold", "release", "evict", "prio"]), seqs,
                         st.integers(0, 6)), min_size=1, max_size=40)


def _call(fn, *a):
    try:
        r = fn(*a)
    except (rdx.RdxError, CacheError) as e:
        return ("err", e.code)
    if isinstance(r, tuple):
        return ("ok", tuple(list(map(int, x)) if isinstance(x, (list, np.ndarray)) else x for x in r))
    if isinstance(r, np.ndarray):
        return ("ok", list(map(int, r)))
    return ("ok", r)


@SETTINGS
@given(ops=ops, slots=st.integers(4, 24), unit=st.sampled_from([1, 2]),
       policy=st.sampled_from(["lru", "lfu", "slru", "priority"]))
def test_tree_equals_the_oracle(ops, slots, unit, policy):
    tree, model = rdx.Tree(slots, unit, policy), TokenTrieCache(slots, unit, policy)
    held = []
    for op, seq, x in ops:
        if op == "prio":
            tree.set_priority(x)
            model.set_priority(x)
        elif op == "evict":
            assert _call(tree.evict, x) == _call(model.evict, x)
        elif op == "release" and held:
            seq_h, m, node, row = held.pop(x % len(held))
            a, b = _call(tree.insert, seq_h, row), _call(model.insert, seq_h, row)
            assert a == b
            if b[0] == "ok":
                k = b[1][0]
                assert _call(tree.free, row[m:k]) == _call(model.free, row[m:k])
            assert _call(tree.unlock, node) == _call(model.unlock, node)
        else:
            a, b = _call(tree.match_prefix, seq), _call(model.match_prefix, seq)
            assert a == b
            m, slots_m, node = b[1]
            assert _call(tree.lock, node) == _call(model.lock, node)
            a, b = _call(tree.alloc, len(seq) - m), _call(model.alloc, len(seq) - m)
            assert a == b
            if b[0] == "err":
                assert _call(tree.unlock, node) == _call(model.unlock, node)
                continue
            row = list(slots_m) + list(b[1])
            if op == "hold":
                held.append((seq, m, node, row))
            else:
                k = model.insert(seq, row)[0]
                assert tree.insert(seq, row)[0] == k
                tree.free(row[m:k])
                model.free(row[m:k])
                tree.unlock(node)
                model.unlock(node)
        assert tree.stats() == model.stats()


groups_st = st.lists(st.tuples(st.integers(0, 30), st.lists(st.tuples(st.integers(1, 20), st.integers(0, 6)),
                                                            min_size=1, max_size=5)), min_size=1, max_size=5)


@SETTINGS
@given(gs=groups_st, s_chunk=st.integers(1, 16), extra=st.integers(0, 200))
def test_batcher_equals_the_oracle(gs, s_chunk, extra):
    groups = [Group(p, tuple(d for d, _ in ms), tuple(t for _, t in ms)) for p, ms in gs]
    m = 2 * s_chunk + extra
    offs = np.concatenate([[0], np.cumsum([len(g.distinct) for g in groups])]).astype(np.int32)
    b = rdx.Batcher([g.prefix_len for g in groups], offs, [d for g in groups for d in g.distinct],
                    [t for g in groups for t in g.decode], s_chunk, m)
    ours = []
    while True:
        e = b.next()
        if len(e) == 0:
            break
        ours.append([(int(k), int(g), -1 if mm < 0 else int(mm - offs[g]), int(bg), int(c)) for k, g, mm, bg, c in e])
    assert ours == batch_iterations(groups, s_chunk, m)


prompts_st = st.lists(st.lists(st.integers(0, 2), min_size=0, max_size=9), min_size=1, max_size=10)


@SETTINGS
@given(prompts=prompts_st)
def test_prefix_groups_equal_the_oracle(prompts):
    g, p, ng, proc = rdx.prefix_groups(prompts)
    total, og, op = min_processed(prompts)
    assert (proc, list(g), list(p), ng) == (total, og, op, len(set(og)))


@SETTINGS
@given(warm=prompts_st, prompts=prompts_st, slots=st.integers(8, 40), unit=st.sampled_from([1, 2]),
       cut=st.integers(0, 12))
def test_schedule_equals_the_oracle(warm, prompts, slots, unit, cut):
    tree, model = rdx.Tree(slots, unit), TokenTrieCache(slots, unit)
    for w in warm:   # served as requests: match, lock, allocate, insert, free, unlock
        m, s, node = model.match_prefix(w)
        tree.match_prefix(w)
        model.lock(node)
        tree.lock(node)
        try:
            new = model.alloc(len(w) - m)
        except CacheError:
            model.unlock(node)
            tree.unlock(node)
            continue
        tree.alloc(len(w) - m)
        k = model.insert(w, list(s) + new)[0]
        tree.insert(w, list(s) + new)
        model.free(new[: k - m])
        tree.free(new[: k - m])
        model.unlock(node)
        tree.unlock(node)
    order, scores = tree.schedule(prompts, fcfs_above=cut)
    o_order, o_scores = osch.lpm_order(model, prompts, fcfs_above=cut)
    assert (list(order), list(scores)) == (o_order, o_scores)

"""Pins of the oracle's token batching (oracle/token_batching.py).

A worked example derived by hand from the BatchLLM explainer's rules, the
closed form of the unbounded case, and properties any run must have (every
token once and in order, prefix before distinct prompt before decode, every
decoding request served every iteration, the memory bound with the stop at
the first chunk that does not fit, queue priority), checked on random
groups by code that reconstructs the state from the output alone."""
import numpy as np
import pytest

from oracle.token_batching import DECODE, DISTINCT, PREFIX, Group, batch_iterations, group_order


def test_worked_example():
    # g0: prefix 4, members (distinct 2, decode 1) and (distinct 3, decode 2)
    # g1: prefix 2, one member (distinct 1, decode 3)
    # prefill tokens 9 and 3 -> R_group 1/9 < 1/3: g1 first.  s_chunk 3, M 12.
    groups = [Group(4, (2, 3), (1, 2)), Group(2, (1,), (3,))]
    assert group_order(groups) == [1, 0]
    its = batch_iterations(groups, 3, 12)
    assert its == [
        # nothing decodes (memory 0): prefix of g1 (2 tokens, memory 4), then
        # 3 of g0's 4 prefix tokens (memory 10)
        [(PREFIX, 1, -1, 0, 2), (PREFIX, 0, -1, 0, 3)],
        # g1's prefix is done: its member's distinct prompt (1 token) comes
        # before the rest of g0's prefix
        [(DISTINCT, 1, 0, 2, 1), (PREFIX, 0, -1, 3, 1)],
        # g1/0 decodes (context 3 -> memory 6); g0/0's 2 tokens fit (10),
        # g0/1's 3 tokens would make 16 > 12: stop
        [(DECODE, 1, 0, 3, 1), (DISTINCT, 0, 0, 4, 2)],
        # two decoding requests: 2*4 + 2*6 = 20 > 12, no chunk
        [(DECODE, 1, 0, 4, 1), (DECODE, 0, 0, 6, 1)],
        # g0/0 generated its one token; g1/0 context 5 -> 10, +6 > 12
        [(DECODE, 1, 0, 5, 1)],
        # nothing decodes: g0/1's prompt fits
        [(DISTINCT, 0, 1, 4, 3)],
        [(DECODE, 0, 1, 7, 1)],
        [(DECODE, 0, 1, 8, 1)],
    ]


def test_shared_prefix_counts_once_in_the_decoding_memory():
    # one group: prefix 4; members (distinct 1, decode 2) x 2 and (distinct 3,
    # decode 1); s_chunk 2, M 14
    groups = [Group(4, (1, 1, 3), (2, 2, 1))]
    its = batch_iterations(groups, 2, 14)
    assert its == [
        [(PREFIX, 0, -1, 0, 2)],
        [(PREFIX, 0, -1, 2, 2)],
        # memory 2 + 2 + 4 = 8
        [(DISTINCT, 0, 0, 4, 1), (DISTINCT, 0, 1, 4, 1), (DISTINCT, 0, 2, 4, 2)],
        # two decoding requests of the group: prefix once (8) + own tokens
        # (2 + 2) = 12; the last distinct token fits (14).  Counting the
        # prefix per request (20) would leave it out.
        [(DECODE, 0, 0, 5, 1), (DECODE, 0, 1, 5, 1), (DISTINCT, 0, 2, 6, 1)],
        [(DECODE, 0, 0, 6, 1), (DECODE, 0, 1, 6, 1), (DECODE, 0, 2, 7, 1)],
    ]


def test_unbounded_memory_closed_form():
    """Memory never binds and a chunk holds any prompt: iteration 0 takes
    every prefix, iteration 1 every distinct prompt, then max(decode)
    iterations of decode tokens."""
    rng = np.random.default_rng(5)
    groups = [Group(int(rng.integers(1, 30)), tuple(int(x) for x in rng.integers(1, 20, k)),
                    tuple(int(x) for x in rng.integers(0, 6, k))) for k in (3, 1, 4, 2)]
    its = batch_iterations(groups, 1000, 10 ** 9)
    order = group_order(groups)
    assert its[0] == [(PREFIX, g, -1, 0, groups[g].prefix_len) for g in order]
    assert its[1] == [(DISTINCT, g, j, groups[g].prefix_len, d) for g in order for j, d in enumerate(groups[g].distinct)]
    t_max = max(max(g.decode) for g in groups)
    assert len(its) == 2 + t_max
    for t in range(t_max):
        assert its[2 + t] == [(DECODE, g, j, groups[g].prefix_len + groups[g].distinct[j] + t, 1)
                              for g in order for j in range(len(groups[g].distinct)) if groups[g].decode[j] > t]


def test_empty_prefix_starts_with_distinct_prompts():
    its = batch_iterations([Group(0, (2, 3), (1, 1))], 4, 100)
    assert its[0] == [(DISTINCT, 0, 0, 0, 2), (DISTINCT, 0, 1, 0, 3)]


def test_minimum_threshold_takes_one_chunk_when_nothing_decodes():
    its = batch_iterations([Group(5, (3,), (0,))], 2, 4)
    # prefix 5 in chunks 2, 2, 1, then distinct 2, 1 -- one chunk each
    assert its == [[(PREFIX, 0, -1, 0, 2)], [(PREFIX, 0, -1, 2, 2)], [(PREFIX, 0, -1, 4, 1)],
                   [(DISTINCT, 0, 0, 5, 2)], [(DISTINCT, 0, 0, 7, 1)]]


def test_bad_parameters():
    with pytest.raises(ValueError):
        batch_iterations([Group(1, (1,), (1,))], 4, 7)
    with pytest.raises(ValueError):
        batch_iterations([Group(1, (0,), (1,))], 4, 8)


def _check_run(groups, s_chunk, m, its):
    """Properties of a run, from the output and the inputs only."""
    order = group_order(groups)
    pre_next = {g: 0 for g in order}                  # next prefix position
    pre_end_it = {g: (-1 if groups[g].prefix_len == 0 else None) for g in order}
    own_next = {(g, j): groups[g].prefix_len for g in order for j in range(len(groups[g].distinct))}
    prompt_end_it = {}
    gen = {k: 0 for k in own_next}
    for it, batch in enumerate(its):
        kinds = [e[0] for e in batch]
        # decode entries first
        assert kinds == sorted(kinds, key=lambda k: k != DECODE)
        dec = [e for e in batch if e[0] == DECODE]
        chunks = [e for e in batch if e[0] != DECODE]
        # every request decoding at this iteration gets exactly one token
        want = sorted(k for k in own_next if k in prompt_end_it and prompt_end_it[k] < it
                      and gen[k] < groups[k[0]].decode[k[1]])
        assert sorted((g, j) for _, g, j, _, _ in dec) == want
        mem = 2 * sum(groups[g].prefix_len for g in {g for g, _ in want}) + \
            sum(2 * (groups[g].distinct[j] + gen[(g, j)]) for g, j in want)
        # pending items at the start of the iteration, in queue order
        pending = []
        for g in order:
            if pre_end_it[g] is not None and pre_end_it[g] < it:
                for j, d in enumerate(groups[g].distinct):
                    if own_next[(g, j)] < groups[g].prefix_len + d:
                        pending.append((DISTINCT, g, j))
        for g in order:
            if pre_next[g] < groups[g].prefix_len:
                pending.append((PREFIX, g, -1))
        # the chunks taken are the first pending items, each the next
        # min(s_chunk, remaining) tokens, within the memory bound ...
        assert [(k, g, j) for k, g, j, _, _ in chunks] == pending[: len(chunks)]
        for k, g, j, begin, c in chunks:
            if k == PREFIX:
                rem = groups[g].prefix_len - pre_next[g]
                assert begin == pre_next[g]
            else:
                rem = groups[g].prefix_len + groups[g].distinct[j] - own_next[(g, j)]
                assert begin == own_next[(g, j)]
            assert c == min(s_chunk, rem)
            mem += 2 * c
            assert mem <= m
        # ... and the next pending item did not fit
        if len(chunks) < len(pending):
            k, g, j = pending[len(chunks)]
            rem = (groups[g].prefix_len - pre_next[g]) if k == PREFIX else \
                (groups[g].prefix_len + groups[g].distinct[j] - own_next[(g, j)])
            assert mem + 2 * min(s_chunk, rem) > m
        assert dec or chunks
        for k, g, j, begin, c in batch:
            if k == DECODE:
                assert begin == groups[g].prefix_len + groups[g].distinct[j] + gen[(g, j)] and c == 1
                gen[(g, j)] += 1
            elif k == DISTINCT:
                own_next[(g, j)] += c
                if own_next[(g, j)] == groups[g].prefix_len + groups[g].distinct[j]:
                    prompt_end_it[(g, j)] = it
            else:
                pre_next[g] += c
                if pre_next[g] == groups[g].prefix_len:
                    pre_end_it[g] = it
    # every token exactly once
    assert all(pre_next[g] == groups[g].prefix_len for g in order)
    assert all(own_next[k] == groups[k[0]].prefix_len + groups[k[0]].distinct[k[1]] for k in own_next)
    assert all(gen[k] == groups[k[0]].decode[k[1]] for k in gen)
    # prefixes start in group order
    starts = []
    for batch in its:
        for k, g, _, _, _ in batch:
            if k == PREFIX and g not in starts:
                starts.append(g)
    assert starts == [g for g in order if groups[g].prefix_len > 0]


@pytest.mark.parametrize("seed", range(30))
def test_random_runs_have_the_properties(seed):
    rng = np.random.default_rng(seed)
    n_groups = int(rng.integers(1, 6))
    groups = []
    for _ in range(n_groups):
        k = int(rng.integers(1, 6))
        groups.append(Group(int(rng.integers(0, 40)), tuple(int(x) for x in rng.integers(1, 25, k)),
                            tuple(int(x) for x in rng.integers(0, 8, k))))
    s_chunk = int(rng.integers(1, 20))
    m = 2 * s_chunk + int(rng.integers(0, 300))
    _check_run(groups, s_chunk, m, batch_iterations(groups, s_chunk, m))


def test_the_checker_catches_a_planted_mistake():
    """A run with one chunk dropped from an iteration fails the checker."""
    groups = [Group(4, (2, 3), (1, 2)), Group(2, (1,), (3,))]
    its = batch_iterations(groups, 3, 12)
    _check_run(groups, 3, 12, its)
    bad = [list(b) for b in its]
    bad[0] = bad[0][:1]
    with pytest.raises(AssertionError):
        _check_run(groups, 3, 12, bad)

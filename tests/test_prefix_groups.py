"""rdx_prefix_groups (the C++ global prefix analysis) against the oracle's
min_processed: N_processed, every group id and prefix length equal on random
batches (duplicates, prompts that are prefixes of others, empty prompts),
the gain-versus-penalty cases and the workload shapes; error paths."""
import numpy as np
import pytest

from oracle.prefix_groups import min_processed
from prefix_shared_kv_token_amd import rdx
from workloads import CONFIGS, Workload


def _same(prompts):
    g, p, ng, proc = rdx.prefix_groups(prompts)
    total, og, op = min_processed(prompts)
    assert proc == total
    assert list(g) == og and list(p) == op
    assert ng == len(set(og))
    return g, p, proc


@pytest.mark.parametrize("seed", range(60))
def test_random_batches(seed):
    rng = np.random.default_rng(500 + seed)
    n = int(rng.integers(1, 14))
    vocab = 2 + seed % 4
    prompts = [[int(x) for x in rng.integers(0, vocab, int(rng.integers(0, 12)))] for _ in range(n)]
    if seed % 3 == 0 and n > 1:
        prompts[-1] = list(prompts[0])                  # a duplicate
    if seed % 4 == 1 and n > 1 and len(prompts[1]) > 2:
        prompts.append(prompts[1][:2])                  # a prefix of another prompt
    _same(prompts)


@pytest.mark.parametrize("t_c,t1,n1", [(10, 4, 4), (12, 4, 4), (11, 4, 4), (3, 2, 3), (4, 2, 3)])
def test_gain_versus_penalty_cases(t_c, t1, n1):
    c = [1] * t_c
    prompts = [c + [2] + [3] * (t1 - 1) + [10 + i] for i in range(n1)] + [c + [4, 5, 5, 20]]
    _same(prompts)


@pytest.mark.parametrize("cfg", [c for c in CONFIGS], ids=lambda c: c.name)
def test_workload_shapes(cfg):
    """Every workload's leaf prompts in a shuffled order: equal to the oracle
    where it is quick, else the closed form (groups at the top-level
    prefixes of the two-level shapes)."""
    wl = Workload(cfg)
    rng = np.random.default_rng(cfg.index)
    leaves = wl.leaf_requests
    order = rng.permutation(len(leaves))
    prompts = [wl.prompt_tokens(leaves[i]) for i in order]
    if sum(len(p) for p in prompts) <= 60000:
        _same([list(map(int, p)) for p in prompts])
    g, p, ng, proc = rdx.prefix_groups(prompts)
    if cfg.n_levels == 2:
        (fan0, l0), (fan1, l1) = cfg.levels
        assert ng == fan0 and set(p.tolist()) == {l0}
        assert proc == fan0 * l0 + fan0 * fan1 * l1
        # members of a group are exactly the leaves under one top-level node
        top = [leaves[i].path[0] for i in order]
        assert len({(a, b) for a, b in zip(g.tolist(), top)}) == fan0


def test_errors():
    l = rdx.lib()
    t = np.zeros(2, np.int32)
    off = np.array([0, 2, 1], np.int64)
    g, pr = np.empty(2, np.int32), np.empty(2, np.int64)
    ng, proc = rdx.i32(), rdx.i64()
    import ctypes
    rc = l.rdx_prefix_groups(2, rdx._p32(t), off.ctypes.data_as(rdx.i64p), rdx._p32(g), pr.ctypes.data_as(rdx.i64p),
                             ctypes.byref(ng), ctypes.byref(proc))
    assert rc == rdx.EINVAL
    assert rdx.prefix_groups([]) [2:] == (0, 0)

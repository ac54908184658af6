"""rdx_batcher (the C++ token batching) against the oracle's
batch_iterations: every iteration's entries equal, bit for bit, on the
hand-worked job, random jobs (empty prefixes, zero decode lengths, tight and
loose memory thresholds) and a full-size BatchLLM-shaped job; error paths."""
import numpy as np
import pytest

from oracle.token_batching import Group, batch_iterations
from prefix_shared_kv_token_amd import rdx


def _product_iterations(groups, s_chunk, m):
    offs = np.concatenate([[0], np.cumsum([len(g.distinct) for g in groups])]).astype(np.int32)
    b = rdx.Batcher([g.prefix_len for g in groups], offs, [d for g in groups for d in g.distinct],
                    [t for g in groups for t in g.decode], s_chunk, m)
    out = []
    while True:
        e = b.next()
        if len(e) == 0:
            return out
        # member index back to (group, index in group)
        out.append([(int(k), int(g), -1 if mm < 0 else int(mm - offs[g]), int(bg), int(c))
                    for k, g, mm, bg, c in e])


def test_worked_example():
    groups = [Group(4, (2, 3), (1, 2)), Group(2, (1,), (3,))]
    assert _product_iterations(groups, 3, 12) == batch_iterations(groups, 3, 12)


@pytest.mark.parametrize("seed", range(40))
def test_random_jobs_equal_the_oracle(seed):
    rng = np.random.default_rng(1000 + seed)
    groups = []
    for _ in range(int(rng.integers(1, 8))):
        k = int(rng.integers(1, 7))
        groups.append(Group(int(rng.integers(1, 50)) if rng.random() > 0.25 else 0,
                            tuple(int(x) for x in rng.integers(1, 30, k)),
                            tuple(int(x) for x in rng.integers(0, 9, k))))
    s_chunk = int(rng.integers(1, 24))
    m = 2 * s_chunk + int(rng.integers(0, 400))
    assert _product_iterations(groups, s_chunk, m) == batch_iterations(groups, s_chunk, m)


def test_batchllm_shaped_job():
    """64 groups of 16 (prefix 2,000, distinct 200, 64 decode tokens), chunks
    of 512, memory for a quarter of the job's KV."""
    groups = [Group(2000, (200,) * 16, (64,) * 16) for _ in range(64)]
    m = 2 * 64 * (2000 + 16 * (200 + 64)) // 4
    ours = _product_iterations(groups, 512, m)
    assert ours == batch_iterations(groups, 512, m)
    assert sum(c for it in ours for (_, _, _, _, c) in it) == 64 * (2000 + 16 * (200 + 64))


def test_errors_and_small_buffer():
    with pytest.raises(rdx.RdxError):
        rdx.Batcher([1], [0, 1], [1], [1], 4, 7)          # threshold < 2 s_chunk
    with pytest.raises(rdx.RdxError):
        rdx.Batcher([1], [0, 0], [], [], 4, 8)            # group without members
    with pytest.raises(rdx.RdxError):
        rdx.Batcher([1], [0, 1], [0], [1], 4, 8)          # empty distinct prompt
    b = rdx.Batcher([4, 2], [0, 2, 3], [2, 3, 1], [1, 2, 3], 3, 12)
    import ctypes
    n = rdx.i32()
    buf = np.zeros((1, 5), np.int32)
    rc = rdx.lib().rdx_batcher_next(b._h, buf.ctypes.data, 1, ctypes.byref(n))
    assert rc == rdx.ENOBUFS and n.value == 2
    # nothing consumed: the first iteration is still the full one
    assert [tuple(r) for r in b.next().tolist()] == [(2, 1, -1, 0, 2), (2, 0, -1, 0, 3)]

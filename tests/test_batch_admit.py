"""Batch admission and completion (rdx_admit / rdx_finish through
Runtime.admit_tokens / Runtime.finish) against the oracle's request-by-request
cache model: whole workloads on the CPU, decode steps simulated on the host
(one slot per request per step, as the decode path allocates them).  Matched
lengths, locked nodes, page-table rows and the final tree statistics must be
bit-identical; a failing admission must leave no lock or slot behind."""
import numpy as np
import pytest

from oracle.run import run_workload
from prefix_shared_kv_token_amd import rdx
from prefix_shared_kv_token_amd.driver import WorkloadRun
from prefix_shared_kv_token_amd.runtime import Runtime
from workloads import Workload, config_by_name

CASES = [
    ("batchllm", dict(levels=((3, 70), (4, 9)), decode_steps=3)),
    ("multilevel", dict(levels=((1, 40), (3, 20), (2, 7)), decode_steps=5)),
    ("helpdesk", dict(levels=((5, 17),), decode_steps=2)),       # no sharing at all
    ("batchllm", dict(levels=((2, 30), (1, 4)), decode_steps=0)),  # a prefix reached by one request
]


def _phases(cfg_name, kw):
    cfg = config_by_name(cfg_name).replace(**kw)
    wl = Workload(cfg)
    rt = Runtime(cfg.dtype, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.total_tokens(),
                 max(len(ph.requests) for ph in wl.phases), cfg.max_seq_len, device="cpu")
    return wl, rt


@pytest.mark.parametrize("name,kw", CASES, ids=[f"{n}-{i}" for i, (n, _) in enumerate(CASES)])
def test_batch_admit_finish_matches_oracle(name, kw):
    wl, rt = _phases(name, kw)
    cfg = wl.cfg
    ref = run_workload(wl, attention_for=())
    gen = wl.decode_token_matrix()
    for pi, ph in enumerate(wl.phases):
        prompts = [wl.prompt_tokens(r) for r in ph.requests]
        b = rt.admit(prompts)
        assert b.matched.tolist() == [ref.matched[r.rid] for r in ph.requests]
        assert b.nodes.tolist() == [ref.node[r.rid] for r in ph.requests]
        leaf = pi == len(wl.phases) - 1
        if leaf:
            for _ in range(cfg.decode_steps):  # host-side stand-in for rdx_decode_step's bookkeeping
                slots = rt.tree.alloc(len(b)).copy()
                pos = rt._rs.kv_len[b.rows64].astype(np.int64)
                rt.host_pt[b.rows64, pos] = slots
                rt._rs.kv_len[b.rows64] += 1
        for r, req in zip(b, ph.requests):
            np.testing.assert_array_equal(rt.host_pt[r.row, : r.kv_len], ref.rows[req.rid])
        rt.finish(b, gen if leaf and cfg.decode_steps else None)
        assert b.kv_len.tolist() == [len(ref.rows[r.rid]) for r in ph.requests]
    assert rt.tree.stats() == ref.stats


def test_driver_phase_arrays_match_per_request_path():
    """The driver's precomputed phase arrays give the same rows as admitting
    prompt lists."""
    cfg = config_by_name("multilevel").replace(levels=((1, 30), (2, 12), (3, 5)), decode_steps=2)
    wl = Workload(cfg)
    run = WorkloadRun.__new__(WorkloadRun)  # host-side fields only (no device inputs)
    run.wl, run.cfg = wl, cfg
    WorkloadRun._phase_arrays(run)
    for pi, ph in enumerate(wl.phases):
        toks = np.concatenate([wl.prompt_tokens(r) for r in ph.requests])
        np.testing.assert_array_equal(run.ptok[pi], toks)
        assert run.poff[pi][-1] == len(toks)
        assert run.expect[pi].tolist() == [r.prompt_len - r.own_len for r in ph.requests]


def test_failed_admission_releases_earlier_requests():
    """A pool too small for the batch: rdx_admit stops at the first request it
    cannot serve; the runtime unlocks and frees the ones admitted before it,
    so the tree is as if nothing had been admitted (apart from LRU stamps)."""
    cfg = config_by_name("batchllm").replace(levels=((1, 20), (4, 10)), decode_steps=0)
    wl = Workload(cfg)
    rt = Runtime(cfg.dtype, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, 45, 8, cfg.max_seq_len, device="cpu")
    hint = rt.admit([wl.prompt_tokens(wl.phases[0].requests[0])])
    rt.finish(hint)
    before = rt.tree.stats()
    with pytest.raises(rdx.RdxError) as e:
        rt.admit([wl.prompt_tokens(r) for r in wl.phases[1].requests])  # needs 4 x 10 > 25 free
    assert e.value.code == rdx.ENOSPC
    after = rt.tree.stats()
    for k in ("free", "cached", "private", "evictable"):
        assert after[k] == before[k], (k, before, after)
    assert len(rt.free_rows) == 8

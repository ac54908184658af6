"""The mixed (token-batched) job on the host: the oracle's cache run over
the batcher's iterations has the properties of an exactly sized pool, and
the product's runner processes the oracle's iterations' tokens, each once."""
import numpy as np
import pytest

from oracle.mixed_run import mixed_groups, run_mixed
from oracle.token_batching import batch_iterations
from workloads import Config, Workload, decode_lengths

# small two-level shapes (groups, members per group, lengths) whose runs mix
# decode tokens and prefill chunks in many iterations
MIX_FP32 = Config("mixed-fp32", 10, 4, 2, 64, "fp32", 1.0, ((6, 40), (3, 20)), 5)
MIX_BF16 = Config("mixed-bf16", 11, 8, 2, 128, "bf16", 0.5, ((5, 300), (4, 40)), 6)
MIX_ARGS = {"mixed-fp32": (64, 262), "mixed-bf16": (256, 948)}


@pytest.mark.parametrize("cfg,s_chunk,m", [(MIX_FP32, 64, 262), (MIX_FP32, 7, 14), (MIX_BF16, 256, 948)])
def test_oracle_mixed_cache_run(cfg, s_chunk, m):
    wl = Workload(cfg)
    tlen = decode_lengths(wl)
    res = run_mixed(wl, s_chunk, m, tlen)
    groups, members = mixed_groups(wl, tlen)
    pre = wl.phases[0].requests
    seen = []
    for g, p in enumerate(pre):
        assert res["matched"][p.rid] == 0
        prow = res["rows"][p.rid]
        assert len(prow) == groups[g].prefix_len
        seen += list(prow)
        for r in members[g]:
            row = res["rows"][r.rid]
            assert res["matched"][r.rid] == groups[g].prefix_len
            assert len(row) == r.prompt_len + groups[g].decode[members[g].index(r)]
            np.testing.assert_array_equal(row[: groups[g].prefix_len], prow)
            seen += list(row[groups[g].prefix_len:])
    # every logical token holds one slot, the smallest free ones first
    used = cfg.total_tokens() - (cfg.decode_steps * len(wl.leaf_requests) - int(tlen.sum()))
    assert sorted(int(x) for x in seen) == list(range(used))
    st = res["stats"]
    assert st["cached"] == used and st["free"] == cfg.total_tokens() - used and st["private"] == 0
    # the batching is interleaved: some iteration holds decode tokens and chunks
    if s_chunk > 7:
        assert any(any(e[0] == 0 for e in it) and any(e[0] != 0 for e in it) for it in res["iterations"])


def test_runner_processes_the_oracle_iterations():
    from prefix_shared_kv_token_amd.mixed import MixedRun

    wl = Workload(MIX_BF16)
    tlen = decode_lengths(wl)
    run = MixedRun(wl, 256, 948, tlen, device="cpu", stage=False)
    groups, members = mixed_groups(wl, tlen)
    its = batch_iterations(groups, 256, 948)
    ours = [[(int(k), int(g), -1 if m < 0 else int(m - run.member_offsets[g]), int(b), int(c))
             for k, g, m, b, c in e] for e in run.iterations]
    assert ours == its
    req, pos = run.job_sources()
    pairs = sorted(zip(req.tolist(), pos.tolist()))
    want = []
    for r in range(run.G + run.M):
        start = 0 if r < run.G else int(run.prefix_len[run.member_group[r - run.G]])
        want += [(r, p) for p in range(start, int(run.req_total_len[r]))]
    assert pairs == sorted(want)


@pytest.mark.parametrize("cfg,s_chunk,m", [(MIX_FP32, 64, 262), (MIX_FP32, 7, 14), (MIX_BF16, 256, 948)])
def test_runner_host_path_matches_the_oracle(cfg, s_chunk, m, monkeypatch):
    """The runner's host side (batcher, admissions, decode slots, plans,
    finishes) with the device launch replaced by the plan build alone:
    every iteration's plan is accepted and every request's matched length
    and page-table row equal the oracle's, bit for bit."""
    import torch
    from prefix_shared_kv_token_amd.mixed import MixedRun

    wl = Workload(cfg)
    tlen = decode_lengths(wl)
    run = MixedRun(wl, s_chunk, m, tlen, device="cpu", stage=False)
    rt = run.rt
    built = []

    def plan_only(kind, reqs, q_len, new_slots, q, k, v, o, timer=None):
        plan = rt.plans[kind]
        plan.build(rt.tree, reqs.nodes, reqs.rows, reqs.kv_len, q_len, reqs.written, new_slots, rt.ld)
        built.append(plan.info()["num_new"])
        rt._rs.written[reqs.rows64] = rt._rs.kv_len[reqs.rows64]

    monkeypatch.setattr(rt, "_launch", plan_only)
    run.q = run.k = run.v = run.o = torch.empty((run.n_tokens, 1))
    run.run(keep_rows=True)
    assert built == [int(t) for t in run.iter_tokens]
    ref = run_mixed(wl, s_chunk, m, tlen)
    assert run.matched == ref["matched"]
    assert sorted(run.rows) == sorted(ref["rows"])
    for rid, row in ref["rows"].items():
        np.testing.assert_array_equal(run.rows[rid], row)


@pytest.mark.parametrize("cfg,s_chunk,m", [(MIX_FP32, 64, 262), (MIX_FP32, 7, 14), (MIX_BF16, 256, 948)])
def test_native_job_dry_run_matches_the_oracle(cfg, s_chunk, m):
    """rdx_job_* planning the whole job on the host (no launch): every plan
    builds and every request's matched length and row equal the oracle's."""
    from prefix_shared_kv_token_amd.mixed import MixedRun

    wl = Workload(cfg)
    tlen = decode_lengths(wl)
    run = MixedRun(wl, s_chunk, m, tlen, device="cpu", stage=False)
    run.run_native(keep_rows=True, dry_run=True)
    ref = run_mixed(wl, s_chunk, m, tlen)
    assert run.matched == ref["matched"]
    assert sorted(run.rows) == sorted(ref["rows"])
    for rid, row in ref["rows"].items():
        np.testing.assert_array_equal(run.rows[rid], row)
    # the tree ends holding every request's sequence, nothing locked
    st = run.rt.tree.stats()
    assert st["private"] == 0 and st["evictable"] == st["cached"]


def test_native_job_errors():
    from prefix_shared_kv_token_amd import rdx

    tree = rdx.Tree(64)
    # member sequence length inconsistent with prefix + distinct + decode
    with pytest.raises(rdx.RdxError):
        rdx.Job(tree, [2], [0, 1], [2], [1], 4, 8, [1, 2, 1, 2, 3, 4], [0, 2, 6], 4, 16)
    job = rdx.Job(tree, [2], [0, 1], [2], [1], 4, 8, [1, 2, 1, 2, 3, 4, 5], [0, 2, 7], 4, 16, rdx.JOB_DRY_RUN)
    # complete before prepare is a state error
    with pytest.raises(rdx.RdxError):
        job.complete()


@pytest.mark.parametrize("pool", [300, 420])
def test_native_job_under_eviction_matches_the_oracle(pool):
    """A pool far smaller than the job (the fp32 shape needs 660 slots with
    every finished request kept): admissions evict finished requests'
    tokens, LRU leaf first; rows and matched lengths still equal the
    oracle's, and the tree evicted something."""
    from prefix_shared_kv_token_amd.mixed import MixedRun

    wl = Workload(MIX_FP32)
    tlen = decode_lengths(wl)
    run = MixedRun(wl, 64, 262, tlen, device="cpu", stage=False, num_slots=pool)
    run.run_native(keep_rows=True, dry_run=True)
    ref = run_mixed(wl, 64, 262, tlen, num_slots=pool)
    assert run.matched == ref["matched"]
    for rid, row in ref["rows"].items():
        np.testing.assert_array_equal(run.rows[rid], row)
    assert run.rt.tree.stats()["evictions"] == ref["stats"]["evictions"] > 0


def test_full_batchllm_job_dry_run_matches_the_oracle():
    """The full BatchLLM-shaped token-batched job (64 groups x 16, prefix
    2,000, distinct 200, 1-64 generated tokens; s_chunk 512, M a fifth of
    the job's K/V entries: the benchmarked job) planned through rdx_job_* on
    the host: every one of the 1,088 requests' matched length and page-table
    row equals the oracle's cache run over the oracle's iterations."""
    from prefix_shared_kv_token_amd.mixed import MixedRun
    from workloads import config_by_name

    cfg = config_by_name("batchllm")
    wl = Workload(cfg)
    tlen = decode_lengths(wl)
    total = cfg.total_tokens() - (cfg.decode_steps * len(wl.leaf_requests) - int(tlen.sum()))
    m = 2 * (total // 5)
    run = MixedRun(wl, 512, m, tlen, device="cpu", stage=False)
    run.run_native(keep_rows=True, dry_run=True)
    ref = run_mixed(wl, 512, m, tlen)
    assert len(ref["rows"]) == 64 + 64 * 16
    assert run.matched == ref["matched"]
    assert sorted(run.rows) == sorted(ref["rows"])
    for rid, row in ref["rows"].items():
        np.testing.assert_array_equal(run.rows[rid], row)

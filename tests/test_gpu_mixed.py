"""GPU parity of the mixed (token-batched) job: chunked prefill and decode
tokens of many requests in every attention launch, through the C ABI,
against the fp64 oracle.  Matched lengths and page-table rows bit-exact;
outputs within max-abs 1e-4 (fp32) / 2e-2 (bf16).  The small shapes are
checked on every output; the full BatchLLM-shaped job (the benchmark's
configuration) on sampled tokens the oracle computes one by one."""
import os

import numpy as np
import pytest

from oracle import causal_attention
from oracle.mixed_run import expected_outputs, run_mixed
from workloads import Config, Workload, config_by_name, decode_lengths

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-4, "bf16": 2e-2}
MIX_FP32 = Config("mixed-fp32", 10, 4, 2, 64, "fp32", 1.0, ((6, 40), (3, 20)), 5)
MIX_BF16 = Config("mixed-bf16", 11, 8, 2, 128, "bf16", 0.5, ((5, 300), (4, 40)), 6)


def _run(cfg, s_chunk, m, items=0, native=True, num_slots=None):
    import torch
    from prefix_shared_kv_token_amd.mixed import MixedRun

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    wl = Workload(cfg)
    tlen = decode_lengths(wl)
    print(f"\n[gpu] mixed {cfg.name} s_chunk={s_chunk} M={m} items={items} native={native}", flush=True)
    run = MixedRun(wl, s_chunk, m, tlen, items=items, num_slots=num_slots)
    if native:
        run.run_native(keep_rows=True)
    else:
        run.run(keep_rows=True)
    torch.cuda.synchronize()
    return wl, tlen, run


def _token_starts(run):
    return np.concatenate([np.zeros(run.G, np.int64), run.prefix_len[run.member_group].astype(np.int64)])


@pytest.mark.parametrize("native", [True, False], ids=["rdx_job", "python"])
@pytest.mark.parametrize("cfg,s_chunk,m,items", [(MIX_FP32, 64, 262, 0), (MIX_FP32, 7, 14, 0),
                                                 (MIX_BF16, 256, 948, 0), (MIX_BF16, 64, 400, 48)])
def test_mixed_small_every_output(cfg, s_chunk, m, items, native):
    wl, tlen, run = _run(cfg, s_chunk, m, items, native)
    ref = run_mixed(wl, s_chunk, m, tlen)
    assert run.matched == ref["matched"]
    assert sorted(run.rows) == sorted(ref["rows"])
    for rid, row in ref["rows"].items():
        np.testing.assert_array_equal(run.rows[rid], row)
    exp = expected_outputs(wl)
    req, pos = run.job_sources()
    start = _token_starts(run)
    o = run.o.float().cpu().numpy()
    want = np.stack([exp[int(run.req_rid[r])][p - start[r]] for r, p in zip(req, pos)])
    err = np.abs(o - want).max()
    print(f"[gpu] {len(req)} tokens in {len(run.iterations)} launches, max abs err {err:.3g}", flush=True)
    assert err <= TOL[cfg.dtype]


def _random_mixed(seed):
    """A small seeded token-batched job: 1-6 groups of 2-5 members (the job
    stages its inputs by the workload's groups, and the prefix analysis puts
    a lone member's group at its own edge), prefix
    1-300 and distinct 1-60 tokens, 1-6 decode steps, GQA 1-4, head_dim 64
    or 128, bf16 or fp32, s_chunk 3-256 and M_threshold between 2 s_chunk
    and the job's whole K/V, and an item target from unsplit to tiny."""
    rng = np.random.default_rng(9100 + seed)
    group = int(rng.choice([1, 2, 4]))
    hkv = int(rng.choice([1, 2]))
    dtype = str(rng.choice(["bf16", "fp32"]))
    cfg = Config(f"mixed-rand{seed}", 100 + seed, group * hkv, hkv, int(rng.choice([64, 128])), dtype,
                 0.5 if dtype == "bf16" else 1.0,
                 ((int(rng.integers(1, 7)), int(rng.integers(1, 300))), (int(rng.integers(2, 6)), int(rng.integers(1, 60)))),
                 int(rng.integers(1, 7)))
    s_chunk = int(rng.integers(3, 257))
    total = 2 * cfg.total_tokens()
    m = int(rng.integers(2 * s_chunk, max(2 * s_chunk + 1, total + 1)))
    return cfg, s_chunk, m, int(rng.choice([0, 0, 16, 100000]))


# RDX_RANDOM_SEEDS=N runs seeds 0..N-1 instead (a longer sweep)
@pytest.mark.parametrize("seed", range(int(os.environ.get("RDX_RANDOM_SEEDS", 12))))
def test_mixed_random_every_output(seed):
    """Every output and page-table row of a seeded random token-batched job
    through the library's job runner, against the oracle."""
    cfg, s_chunk, m, items = _random_mixed(seed)
    wl, tlen, run = _run(cfg, s_chunk, m, items)
    ref = run_mixed(wl, s_chunk, m, tlen)
    assert run.matched == ref["matched"]
    for rid, row in ref["rows"].items():
        np.testing.assert_array_equal(run.rows[rid], row)
    exp = expected_outputs(wl)
    req, pos = run.job_sources()
    start = _token_starts(run)
    o = run.o.float().cpu().numpy()
    want = np.stack([exp[int(run.req_rid[r])][p - start[r]] for r, p in zip(req, pos)])
    err = np.abs(o - want).max()
    print(f"[gpu] {cfg.levels} s_chunk={s_chunk} M={m}: {len(req)} tokens in {len(run.iterations)} launches, "
          f"max abs err {err:.3g}", flush=True)
    assert err <= TOL[cfg.dtype]


def test_mixed_under_eviction_every_output():
    """A pool of 300 slots for a job of 660 tokens: admissions evict finished
    requests (the slots of their pages are reused while later launches read
    their own); rows bit-exact, every output within tolerance."""
    wl, tlen, run = _run(MIX_FP32, 64, 262, num_slots=300)
    ref = run_mixed(wl, 64, 262, tlen, num_slots=300)
    assert ref["stats"]["evictions"] > 0
    assert run.matched == ref["matched"]
    for rid, row in ref["rows"].items():
        np.testing.assert_array_equal(run.rows[rid], row)
    exp = expected_outputs(wl)
    req, pos = run.job_sources()
    start = _token_starts(run)
    o = run.o.float().cpu().numpy()
    want = np.stack([exp[int(run.req_rid[r])][p - start[r]] for r, p in zip(req, pos)])
    err = np.abs(o - want).max()
    print(f"[gpu] evicting pool: {len(run.iterations)} launches, max abs err {err:.3g}", flush=True)
    assert err <= TOL["fp32"]


def _token_q(wl, r, pos):
    """Query of request r at position pos (own prompt token or decode token)."""
    own_start = r.prompt_len - r.own_len
    if pos < r.prompt_len:
        return wl.request_q(r)[pos - own_start]
    return wl.decode_q(r)[pos - r.prompt_len]


def test_mixed_batchllm_full_size_sampled():
    """64 groups x 16 (prefix 2,000, distinct 200, up to 64 generated), chunks
    of 512, KV memory bound a fifth of the job's -- as the benchmark runs it.
    Every request's matched length and page-table row against the oracle's
    cache run (bit-exact); outputs on sampled tokens: one from every launch,
    48 more at random, the job's first and last."""
    cfg = config_by_name("batchllm")
    wl = Workload(cfg)
    tlen = decode_lengths(wl)
    total = cfg.total_tokens() - (cfg.decode_steps * len(wl.leaf_requests) - int(tlen.sum()))
    m = 2 * (total // 5)
    wl, tlen, run = _run(cfg, 512, m)
    mixed = sum(1 for e in run.iterations if (e[:, 0] == 0).any() and (e[:, 0] != 0).any())
    assert mixed > 0
    ref = run_mixed(wl, 512, m, tlen)
    assert run.matched == ref["matched"]
    assert sorted(run.rows) == sorted(ref["rows"])
    for rid, row in ref["rows"].items():
        np.testing.assert_array_equal(run.rows[rid], row)
    print(f"[gpu] batchllm mixed: {len(ref['rows'])} rows bit-exact", flush=True)
    req, pos = run.job_sources()
    rng = np.random.default_rng(17)
    per_launch = [int(rng.integers(run.iter_off[i], run.iter_off[i + 1])) for i in range(len(run.iterations))]
    picks = np.unique(np.concatenate([per_launch, rng.choice(len(req), 48, replace=False), [0, len(req) - 1]]))
    reqs = wl.phases[0].requests + wl.phases[1].requests
    by_rid = {r.rid: r for r in reqs}
    kv_cache = {}
    worst = 0.0
    o = run.o
    for i in picks:
        r = by_rid[int(run.req_rid[req[i]])]
        p = int(pos[i])
        if r.rid not in kv_cache:
            kv_cache = {r.rid: wl.request_full_kv(r)}
        k, v = kv_cache[r.rid]
        want = causal_attention(_token_q(wl, r, p)[None], k, v, np.array([p]))[0]
        got = o[int(i)].float().cpu().numpy()
        worst = max(worst, float(np.abs(got - want).max()))
    print(f"[gpu] batchllm mixed: {len(run.iterations)} launches ({mixed} mixed), {len(picks)} sampled tokens, "
          f"max abs err {worst:.3g}", flush=True)
    assert worst <= TOL["bf16"]

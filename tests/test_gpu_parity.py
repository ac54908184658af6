"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Match lengths and page-table rows must be bit-exact; attention outputs
within max-abs 1e-4 (fp32 workloads) or 2e-2 (bf16 workloads, fp32
accumulation).  Small shapes are checked on every output; the five full-size
workloads run exactly as the benchmark runs them and are checked on sampled
requests the oracle computes one by one."""
import os

import numpy as np
import pytest

from oracle import run_workload
from workloads import CONFIGS, Workload, config_by_name

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-4, "bf16": 2e-2}


def _torch():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


def _fragmenter(num_slots, keep, seed):
    def prep(cache):
        rng = np.random.default_rng(seed)
        allslots = np.asarray(cache.alloc(num_slots))
        cache.free(np.sort(rng.choice(allslots, keep, replace=False)))
    return prep


def run_and_check(cfg, sample_leaves=None, extend_items=0, decode_items=0, hole_seed=None, extra_slots=0,
                  poison=False, leaf_extra=(), kv_row_pitch=None):
    """poison: every pool row starts as NaN, so any key or value the kernels
    read that the workload never wrote shows up in the outputs.
    leaf_extra: rids checked besides the sampled leaves (other phases)."""
    torch = _torch()
    from prefix_shared_kv_token_amd.driver import WorkloadRun

    wl = Workload(cfg)
    print(f"\n[gpu] {cfg.name} levels={cfg.levels} Hq/Hkv={cfg.n_q_heads}/{cfg.n_kv_heads} D={cfg.head_dim} "
          f"{cfg.dtype} items={extend_items}/{decode_items} holes={hole_seed}", flush=True)
    run = WorkloadRun(wl, extend_items=extend_items, decode_items=decode_items, hole_seed=hole_seed,
                      extra_slots=extra_slots, kv_row_pitch=kv_row_pitch)
    if poison:
        run.rt.k_pool.fill_(float("nan"))
        run.rt.v_pool.fill_(float("nan"))
        torch.cuda.synchronize()
    out = run.run()
    torch.cuda.synchronize()
    leaves = wl.leaf_requests
    if sample_leaves is None:
        rids = [r.rid for r in wl.all_requests]
    else:
        idx = sorted(set(int(i) % len(leaves) for i in sample_leaves))
        rids = [leaves[i].rid for i in idx] + [wl.phases[0].requests[0].rid] + list(leaf_extra)
    prep = _fragmenter(run.num_slots, cfg.total_tokens(), hole_seed) if hole_seed is not None else None
    ref = run_workload(wl, num_slots=run.num_slots, attention_for=rids, prepare=prep)
    # ---- indices: bit-exact ----
    for pi, ph in enumerate(wl.phases):
        for j, r in enumerate(ph.requests):
            assert out["matched"][pi][j] == ref.matched[r.rid], (pi, j)
            np.testing.assert_array_equal(out["rows"][pi][j], ref.rows[r.rid])
    # ---- outputs ----
    tol = TOL[cfg.dtype]
    worst = 0.0
    for pi, ph in enumerate(wl.phases):
        off = 0
        for j, r in enumerate(ph.requests):
            if r.rid in ref.extend_out:
                got = out["extend"][pi][off:off + r.own_len].float().cpu().numpy()
                err = float(np.abs(got - ref.extend_out[r.rid]).max())
                worst = max(worst, err)
                assert err <= tol, f"extend phase {pi} request {j}: max abs err {err}"
                if r.decode_steps:
                    gd = out["decode"][:, j].float().cpu().numpy()
                    err = float(np.abs(gd - ref.decode_out[r.rid]).max())
                    worst = max(worst, err)
                    assert err <= tol, f"decode request {j}: max abs err {err}"
            off += r.own_len
    print(f"[gpu] {cfg.name}: {len(rids)} requests checked, max abs err {worst:.3g} (tol {tol})", flush=True)
    return run, out, ref


def test_tiny_all_outputs():
    run_and_check(config_by_name("tiny"))


def test_tiny_split_items_and_fragmented_pool():
    cfg = config_by_name("tiny")
    run_and_check(cfg, extend_items=100000, decode_items=100000, hole_seed=5, extra_slots=97)


EDGE = [
    # bf16 head_dim 64, GQA 4, ragged suffix
    ("tiny", dict(levels=((2, 150), (3, 37)), n_q_heads=8, n_kv_heads=2, dtype="bf16", sigma=0.5, decode_steps=5)),
    # one-token suffixes
    ("batchllm", dict(levels=((2, 200), (6, 1)), decode_steps=3)),
    # no shared prefix at all (every request is its own hint), MHA
    ("helpdesk", dict(levels=((5, 77),), n_q_heads=4, n_kv_heads=4, decode_steps=4)),
    # a prefix reached by a single request degrades to its own range
    ("batchllm", dict(levels=((3, 100), (1, 20)), decode_steps=2)),
    # fp32, GQA, three levels
    ("tiny", dict(levels=((1, 40), (3, 17), (2, 9)), n_q_heads=8, n_kv_heads=2, head_dim=128, decode_steps=6)),
    # GQA 8 (group of 8 query heads per KV head)
    ("longprefix", dict(levels=((2, 300), (4, 33)), n_q_heads=16, n_kv_heads=2, decode_steps=3)),
    # 24 leaves x 4 grouped heads = 96 decode rows under one root: one
    # decode tile of two 16-row groups per wave (head_dim 128 and 64)
    ("multilevel", dict(levels=((1, 100), (2, 40), (12, 11)), decode_steps=4)),
    ("tiny", dict(levels=((1, 90), (24, 13)), n_q_heads=8, n_kv_heads=2, dtype="bf16", sigma=0.5, decode_steps=3)),
]


@pytest.mark.parametrize("base,kw", EDGE, ids=[f"{b}-{i}" for i, (b, _) in enumerate(EDGE)])
@pytest.mark.parametrize("items", [0, 100000], ids=["fused", "split"])
def test_edge_shapes(base, kw, items):
    run_and_check(config_by_name(base).replace(**kw), extend_items=items, decode_items=items)


def _random_case(seed):
    """A small seeded workload: 1-3 tree levels of random fan-out and length
    (one-token levels included), GQA group 1-8, head_dim 64 or 128, bf16 or
    fp32, 1-5 decode steps, an item target from unsplit to one block per
    item, and half the time a fragmented pool."""
    rng = np.random.default_rng(7000 + seed)
    depth = int(rng.integers(1, 4))
    levels = []
    for d in range(depth):
        n = int(rng.integers(1, 4 if d < depth - 1 else 6))
        levels.append((n, int(rng.integers(1, 150 if d == 0 else 60))))
    group = int(rng.choice([1, 2, 4, 8]))
    hkv = int(rng.choice([1, 2]))
    dtype = str(rng.choice(["bf16", "bf16", "fp32"]))
    kw = dict(levels=tuple(levels), n_q_heads=group * hkv, n_kv_heads=hkv, head_dim=int(rng.choice([64, 128])),
              dtype=dtype, sigma=0.5 if dtype == "bf16" else 1.0, decode_steps=int(rng.integers(1, 6)))
    items = int(rng.choice([0, 0, 3, 100000]))
    holes = (seed, int(rng.integers(1, 400))) if rng.random() < 0.5 else (None, 0)
    return kw, items, holes


# RDX_RANDOM_SEEDS=N runs seeds 0..N-1 instead (a longer sweep)
@pytest.mark.parametrize("seed", range(int(os.environ.get("RDX_RANDOM_SEEDS", 32))))
def test_random_shapes(seed):
    """Every output of a seeded random workload against the oracle; odd
    seeds start from NaN-filled pools, so a read of any row the workload
    never wrote shows in the outputs."""
    kw, items, (hole_seed, extra) = _random_case(seed)
    run_and_check(config_by_name("tiny").replace(**kw), extend_items=items, decode_items=items,
                  hole_seed=hole_seed, extra_slots=extra, poison=seed % 2 == 1)


def test_short_last_round_cut_into_quarters():
    """Member extend of 5 wide tiles per KV head on 4 items per head: the
    fifth tile runs as 4 quarter pieces merged by LSE; the decode tile is
    split into 4 items.  Every output against the oracle."""
    cfg = config_by_name("helpdesk").replace(levels=((1, 512), (4, 80)), n_q_heads=8, n_kv_heads=2, decode_steps=3)
    run, out, ref = run_and_check(cfg, extend_items=8, decode_items=8)
    info = out["plan_info"][1]
    assert info["num_tiles"] == 5 and info["num_split_tiles"] == 1 and info["num_items"] == 2 * 8


def test_fragmented_pool_bf16():
    cfg = config_by_name("multilevel").replace(levels=((1, 100), (2, 40), (3, 11)), decode_steps=4)
    run_and_check(cfg, hole_seed=11, extra_slots=333, poison=True)


def test_deterministic_and_kv_store_roundtrip():
    torch = _torch()
    from prefix_shared_kv_token_amd.driver import WorkloadRun

    cfg = config_by_name("batchllm").replace(levels=((2, 130), (4, 21)), decode_steps=3)
    wl = Workload(cfg)
    run = WorkloadRun(wl)
    a = run.run()
    b = run.run()
    torch.cuda.synchronize()
    for x, y in zip(a["extend"], b["extend"]):
        assert torch.equal(x, y)
    assert torch.equal(a["decode"], b["decode"])
    # the pool holds every stored token's K/V at its slot
    leaf = wl.leaf_requests[1]
    row = a["rows"][-1][1]
    k_log, v_log = wl.request_full_kv(leaf)
    idx = torch.as_tensor(row, device=run.rt.device).long()
    hd = cfg.n_kv_heads * cfg.head_dim  # a pool row holds the slot's [Hkv][D] first, then padding
    kp = run.rt.k_pool[idx][:, :hd].reshape(len(row), cfg.n_kv_heads, cfg.head_dim).float().cpu().numpy()
    vp = run.rt.v_pool[idx][:, :hd].reshape(len(row), cfg.n_kv_heads, cfg.head_dim).float().cpu().numpy()
    np.testing.assert_array_equal(kp, k_log)
    np.testing.assert_array_equal(vp, v_log)


def test_pool_over_2gib_uses_64bit_addressing():
    """A KV pool of more than 2 GiB per tensor (32 x 128 bf16 heads, ~264k
    slots) takes the kernels' 64-bit address path; the scattered free set puts
    the workload's pages all over it, past the 2 GiB mark.  Every pool row
    starts as NaN: keys past a job's end must not let row 0 (or any other
    unwritten row) into the outputs."""
    row_bytes = 32 * 128 * 2
    extra = (1 << 31) // row_bytes + 4096
    cfg = config_by_name("helpdesk").replace(levels=((1, 60), (6, 20)), decode_steps=3)
    run, _, _ = run_and_check(cfg, hole_seed=21, extra_slots=extra, poison=True)
    assert run.num_slots * row_bytes > (1 << 31)


def test_decode_steps_match_decode_step_calls():
    """Runtime.decode_steps (the stacked step inputs checked once, pointers
    advanced per step) gives bit-identical outputs and page-table rows to
    one decode_step call per step (the path a run with per-step timers
    takes), with one output per step and with one output buffer rewritten
    by every step."""
    torch = _torch()
    from prefix_shared_kv_token_amd.driver import WorkloadRun

    cfg = config_by_name("multilevel").replace(levels=((1, 90), (2, 40), (3, 13)), decode_steps=5)
    run = WorkloadRun(Workload(cfg))
    a = run.run()                    # decode_steps
    b = run.run(timers={})           # decode_step per step
    c = run.run(keep_outputs=False)  # decode_steps, one shared output buffer
    torch.cuda.synchronize()
    assert torch.equal(a["decode"], b["decode"])
    assert torch.equal(a["decode"][-1], c["decode"][0])
    for p, q in zip(a["rows"], b["rows"]):
        for x, y in zip(p, q):
            np.testing.assert_array_equal(x, y)


def test_separate_calls_match_decode_step():
    """The decode path through the separate entry points (rdx_plan_build,
    rdx_plan_upload, rdx_kv_store, rdx_decode_attention; used when launches
    are recorded) gives bit-identical outputs to rdx_decode_step."""
    torch = _torch()
    from prefix_shared_kv_token_amd.driver import WorkloadRun

    cfg = config_by_name("multilevel").replace(levels=((1, 90), (2, 40), (3, 13)), decode_steps=5)
    run = WorkloadRun(Workload(cfg))
    a = run.run()
    b = run.run(record=True)
    torch.cuda.synchronize()
    for x, y in zip(a["extend"], b["extend"]):
        assert torch.equal(x, y)
    assert torch.equal(a["decode"], b["decode"])
    for p, q in zip(a["rows"], b["rows"]):
        for x, y in zip(p, q):
            np.testing.assert_array_equal(x, y)


# Sampled leaves at full size: both sides of every kind of tile boundary.
# Helpdesk: extend tiles of 256 rows (6.4 requests), one 64-row decode tile.
# BatchLLM / Long-prefix: groups of 16 members (a decode tile each); first
# and last member of several groups.  Multi-level: 24 leaves under 8
# branches of 3; decode tiles are cut on branch boundaries (leaves 0-14,
# then 15-23), so leaves 14 and 15 sit on either side of the tile boundary,
# and 15-17 share the branch that opens the second tile.
FULL_SAMPLES = {
    "helpdesk": [0, 6, 7, 31, 32, 63],
    "batchllm": [0, 15, 16, 31, 500, 511, 512, 1008, 1023],
    "longprefix": [0, 15, 16, 31, 32, 47, 48, 63],
    "multilevel": [0, 2, 3, 11, 14, 15, 16, 17, 23],
}


@pytest.mark.parametrize("cfg", [c for c in CONFIGS if c.dtype == "bf16"], ids=lambda c: c.name)
def test_full_size_sampled(cfg):
    """Full-size workloads, default launch configuration (as timed by the
    benchmark), checked on sampled leaf requests, the first hint and, for
    the multi-level tree, the first, a middle and the last branch request
    (the middle phase, whose extend attends the root shared by all 8)."""
    wl = Workload(cfg)
    extra = []
    if len(wl.phases) > 2:
        mid = wl.phases[1].requests
        extra = [mid[0].rid, mid[len(mid) // 2].rid, mid[-1].rid]
    run_and_check(cfg, sample_leaves=FULL_SAMPLES[cfg.name], leaf_extra=extra)


def test_full_size_sampled_pool_over_2gib():
    """BatchLLM at full size with a pool of more than 2 GiB per matrix, so
    extend and decode run their 64-bit offset variants (the addressing of any
    pool sized for a large share of HBM), unused pool rows NaN-poisoned:
    sampled leaves (first and last members of several groups) against the
    oracle."""
    cfg = config_by_name("batchllm")
    row_bytes = cfg.n_kv_heads * cfg.head_dim * 2 + 256   # the recommended padded pitch
    extra = (1 << 31) // row_bytes + 4096
    run, _, _ = run_and_check(cfg, sample_leaves=[0, 15, 16, 511, 512, 1023], extra_slots=extra, poison=True)
    assert run.rt.k_pool.numel() * run.rt.k_pool.element_size() > (1 << 31)


def test_decode_long_items():
    """Decode items of 56+ key blocks (a 3,500-token prefix shared by 4
    requests, one decode item per KV head): every output against the
    oracle, on the 32-bit and the 64-bit (scattered pool over 2 GiB,
    NaN-poisoned) paths."""
    cfg = config_by_name("batchllm").replace(levels=((1, 3500), (4, 9)), decode_steps=3)
    run, _, _ = run_and_check(cfg, decode_items=8)
    assert run.rt._info.num_items == 8   # the last decode step's plan: one item per KV head
    row_bytes = 8 * 128 * 2
    extra = (1 << 31) // row_bytes + 4096
    run_and_check(cfg, decode_items=8, hole_seed=3, extra_slots=extra, poison=True)


@pytest.mark.gpu
@pytest.mark.parametrize("pitch_pad", [0, 8])
@pytest.mark.parametrize("name,levels,decode", [
    ("batchllm", ((3, 150), (5, 70)), 3),
    ("tiny", ((1, 64), (4, 16)), 3),
])
def test_kv_row_pitch(name, levels, decode, pitch_pad):
    """The pools' row pitch is the caller's: dense rows (kv_row_pitch 0) and
    rows padded by 16 bytes (8 bf16 / 4 fp32 elements past Hkv x head_dim)
    give the oracle's outputs through the store, extend (both split modes)
    and decode kernels, with unwritten pool memory poisoned."""
    cfg = config_by_name(name).replace(levels=levels, decode_steps=decode)
    elems = 0 if pitch_pad == 0 else cfg.n_kv_heads * cfg.head_dim + (pitch_pad if cfg.dtype == "bf16" else 4)
    for items in (0, 100000):
        run, _, _ = run_and_check(cfg, extend_items=items, decode_items=items, poison=True, kv_row_pitch=elems)
        assert run.rt.kv_row_pitch == (elems or cfg.n_kv_heads * cfg.head_dim)

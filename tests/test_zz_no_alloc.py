"""rdx_decode_attention_noalloc (through the C ABI) against
rdx_decode_attention on the same plans: bit-identical outputs on two calls
in a row, the second with a smaller input; a plan whose split tiles need
more workspace than the built-in one is rejected before anything runs."""
import numpy as np
import pytest

from workloads import Workload, config_by_name

pytestmark = pytest.mark.gpu


def _decode_launches(cfg, decode_items=0):
    import torch
    from prefix_shared_kv_token_amd.driver import WorkloadRun

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    run = WorkloadRun(Workload(cfg), decode_items=decode_items)
    out = run.run(record=True)
    torch.cuda.synchronize()
    from prefix_shared_kv_token_amd import rdx
    dec = [l for l in out["launches"] if l[0] == rdx.PLAN_DECODE]
    return run, dec


def _check_same(run, launches):
    import torch
    from prefix_shared_kv_token_amd import rdx

    rt = run.rt
    n_split = 0
    for kind, plan, dev, q, o, info in launches:
        ws = rt._workspace(info["workspace_bytes"])
        ref = torch.full_like(o, float("nan"))
        got = torch.full_like(o, float("nan"))
        rdx.decode_attention(rt.desc, plan, dev, q, rt.k_pool, rt.v_pool, rt.page_table, ref, ws, ws.numel())
        rdx.decode_attention_noalloc(rt.desc, plan, dev, q, rt.k_pool, rt.v_pool, rt.page_table, got)
        torch.cuda.synchronize()
        assert torch.equal(ref, got)
        assert torch.equal(ref, o)   # the launch as the run made it
        n_split += info["num_split_tiles"] > 0
    return n_split


def test_noalloc_decode_matches_decode_attention():
    # call 1: 64 requests sharing a 1,000-token prefix, MHA 32 heads: every
    # decode step splits its tile (about 16 MiB of partial states)
    big = config_by_name("helpdesk").replace(decode_steps=2)
    run, dec = _decode_launches(big)
    print(f"\n[gpu] no-alloc decode: {big.levels}, {len(dec)} launches, workspace "
          f"{max(l[5]['workspace_bytes'] for l in dec)} B", flush=True)
    assert _check_same(run, dec) == len(dec)
    del run, dec
    # call 2: a smaller input on the same GPU (the array keeps the previous
    # call's contents; nothing in it needs clearing)
    small = config_by_name("batchllm").replace(levels=((2, 300), (8, 20)), decode_steps=2)
    run, dec = _decode_launches(small, decode_items=64)
    print(f"[gpu] no-alloc decode: {small.levels}, {len(dec)} launches, workspace "
          f"{max(l[5]['workspace_bytes'] for l in dec)} B", flush=True)
    assert _check_same(run, dec) == len(dec)


def test_noalloc_rejects_a_workspace_beyond_the_builtin_one():
    """64 requests over a cached 8,192-token prefix, MHA 32 x 128, every
    64-key block its own work item: 128 pieces x 64 tokens x 32 heads x
    512 B = 128 MiB of partial states, over the 64 MiB built in: EINVAL,
    nothing enqueued (the check precedes every device access)."""
    import torch
    from prefix_shared_kv_token_amd import rdx
    from prefix_shared_kv_token_amd.runtime import Runtime

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    n = 64
    rt = Runtime("bf16", 32, 32, 128, 9000, n, 8300)
    prefix = np.arange(1, 8193, dtype=np.int32)
    rt.finish(rt.admit([prefix]))                      # the prefix is cached
    reqs = rt.admit([np.concatenate([prefix, [50000 + i]]).astype(np.int32) for i in range(n)])
    assert (reqs.matched == 8192).all()
    plan = rdx.Plan(rt.desc, rdx.PLAN_DECODE, 100000)
    plan.build(rt.tree, reqs.nodes, reqs.rows, reqs.kv_len, np.ones(n, np.int32), reqs.written,
               reqs.new_slots[:n], rt.ld)
    info = plan.info()
    assert info["workspace_bytes"] > 64 << 20
    q = torch.zeros((n, 32, 128), dtype=torch.bfloat16, device=rt.device)
    o = torch.empty_like(q)
    dev = torch.zeros(max(info["device_bytes"], 64), dtype=torch.uint8, device=rt.device)
    with pytest.raises(rdx.RdxError) as e:
        rdx.decode_attention_noalloc(rt.desc, plan, dev, q, rt.k_pool, rt.v_pool, rt.page_table, o)
    assert e.value.code == rdx.EINVAL and "workspace" in str(e.value)

"""Launch timing (rdx_timing_begin / rdx_timing_read) on the GPU: one record
per attention launch in launch order, with its plan kind, a positive kernel
duration, and a merge duration exactly where the plan split tiles; a
recording stops at its capacity and the events it created are reused."""
import numpy as np
import pytest

from workloads import Workload, config_by_name

pytestmark = pytest.mark.gpu


def test_timing_records_each_launch():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from prefix_shared_kv_token_amd import rdx
    from prefix_shared_kv_token_amd.driver import WorkloadRun

    # Helpdesk-like tree (2 phases) with a split extend tile and split decode tiles
    cfg = config_by_name("helpdesk").replace(levels=((1, 512), (4, 80)), n_q_heads=8, n_kv_heads=2, decode_steps=3)
    wl = Workload(cfg)
    run = WorkloadRun(wl, extend_items=8, decode_items=8)
    run.run(keep_outputs=False)
    torch.cuda.synchronize()
    n_launch = len(wl.phases) + cfg.decode_steps
    kinds_expected = [rdx.PLAN_EXTEND] * len(wl.phases) + [rdx.PLAN_DECODE] * cfg.decode_steps
    print(f"\n[gpu] timing: {n_launch} launches per pass", flush=True)
    for rep in range(2):  # the second recording reuses the first one's events
        rdx.timing_begin(n_launch)
        out = run.run(keep_outputs=False)
        torch.cuda.synchronize()
        attn, merge, kinds = rdx.timing_read(n_launch)
        assert len(attn) == n_launch
        assert kinds.tolist() == kinds_expected
        assert np.all(attn > 0) and np.all(np.isfinite(attn))
        split = [info["num_split_tiles"] > 0 for info in out["plan_info"]]
        for i, s in enumerate(split):  # extend launches: merge time only where tiles were split
            assert (merge[i] > 0) == s, (i, merge[i], s)
        assert np.all(merge[len(wl.phases):] > 0)  # decode tiles cut into 8 items each
    # a recording stops at its capacity: the launches after it are not recorded
    rdx.timing_begin(2)
    run.run(keep_outputs=False)
    torch.cuda.synchronize()
    attn, merge, kinds = rdx.timing_read(n_launch)
    assert len(attn) == 2 and kinds.tolist() == kinds_expected[:2]

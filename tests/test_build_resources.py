"""The build reads the compiler's per-kernel resource remarks and refuses a
library in which any kernel uses scratch memory (a spill, or a private array
lowered to scratch, slows a kernel several-fold without changing its
results)."""
import os

import pytest

from prefix_shared_kv_token_amd import build

REMARKS = """\
x.h:10:1: remark: Function Name: _ZN3rdx1aEv [-Rpass-analysis=kernel-resource-usage]
x.h:10:1: remark:     VGPRs: 249 [-Rpass-analysis=kernel-resource-usage]
x.h:10:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
x.h:10:1: remark:     Occupancy [waves/SIMD]: 2 [-Rpass-analysis=kernel-resource-usage]
x.h:10:1: remark:     LDS Size [bytes/block]: 108032 [-Rpass-analysis=kernel-resource-usage]
x.h:20:1: remark: Function Name: _ZN3rdx1bEv [-Rpass-analysis=kernel-resource-usage]
x.h:20:1: remark:     VGPRs: 152 [-Rpass-analysis=kernel-resource-usage]
x.h:20:1: remark:     ScratchSize [bytes/lane]: 136 [-Rpass-analysis=kernel-resource-usage]
x.h:20:1: remark:     Dynamic Stack: False [-Rpass-analysis=kernel-resource-usage]
"""


def test_remarks_parsed_per_kernel():
    res = build.kernel_resources(REMARKS)
    assert res["_ZN3rdx1aEv"] == {"VGPRs": 249, "ScratchSize": 0, "Occupancy": 2, "LDS Size": 108032}
    assert res["_ZN3rdx1bEv"]["ScratchSize"] == 136
    assert res["_ZN3rdx1bEv"]["Dynamic Stack"] == "False"


def test_scratch_fails_the_build():
    res = build.kernel_resources(REMARKS)
    with pytest.raises(RuntimeError, match="_ZN3rdx1bEv"):
        build.check_resources(res)
    del res["_ZN3rdx1bEv"]
    build.check_resources(res)


def test_built_library_has_no_scratch():
    """The resource table the last build wrote: every kernel listed, none
    with scratch."""
    if not os.path.exists(build.RESOURCES):
        pytest.skip("library not built here")
    lines = open(build.RESOURCES).read().splitlines()
    names = [l.split()[0] for l in lines]
    for k in ("attn_bf16_wide_kernel", "attn_decode_kernel", "merge_kernel", "kv_store_kernel", "step_store_kernel"):
        assert any(k in n for n in names), k
    assert all(" ScratchSize=0 " in l + " " for l in lines), [l for l in lines if "ScratchSize=0" not in l]

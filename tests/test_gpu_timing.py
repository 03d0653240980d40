"""The library's per-kernel timing: all kernels, or only the named ones."""
import pytest
import torch

import sparse_mixture_experts_capacity_amd as moe
from gpu_helpers import DEV, Run, config_for, say
from workloads import Workload

pytestmark = pytest.mark.gpu


def test_timing_only_named_kernels():
    w = Workload("timing", T=300, d=128, F=128, E=8, k=2, capacity_factor=1.25)
    say("[timing] all kernels, then ffn1_swiglu only")
    run = Run(w)
    cfg = config_for(w, bias=run.bias, stream=None)
    ws = moe.Workspace(moe.moe_workspace_size(cfg))
    ws.bind(cfg)
    out = torch.empty((w.T, w.d), dtype=w.torch_dtype, device=DEV)

    def timed_steps(only, n=3):
        moe.moe_timing_reset()
        moe.moe_timing_only(only)
        moe.moe_timing_enable(True)
        for _ in range(n):
            moe.moe_forward(run.x, run.Wg, run.W1, run.W3, run.W2, cfg, out)
        torch.cuda.synchronize()
        moe.moe_timing_enable(False)
        return moe.moe_timing_read()

    every = timed_steps(None)
    assert {"ffn1_swiglu", "ffn2", "combine"} <= set(every)
    assert all(c == 3 and t > 0.0 for c, t in every.values())
    one = timed_steps("ffn1_swiglu")
    assert set(one) == {"ffn1_swiglu"} and one["ffn1_swiglu"][0] == 3
    two = timed_steps(["ffn2", "combine"])
    assert set(two) == {"ffn2", "combine"}
    assert timed_steps("no_such_kernel") == {}
    moe.moe_timing_only(None)

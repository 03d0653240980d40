"""Workspace canaries (a debugging aid of the host layer): with guards after
every workspace region, no kernel of the forward, the routing entry points,
the aux loss or the router backward may write past its region; and a guard
overwritten from the host is reported with the region before it."""
import pytest
import torch

import sparse_mixture_experts_capacity_amd as moe
from gpu_helpers import DEV, Run, config_for, route_buffers, say
from workloads import SKEW_BIAS, SOFTMAX_THEN_TOPK, Workload, random_logits

pytestmark = pytest.mark.gpu

CASES = {
    "long_rows_shared": Workload("cn_long", T=1600, d=192, F=320, E=4, k=1, S=1,
                                 capacity_factor=1.25),
    "wide_drops": Workload("cn_wide", T=1000, d=256, F=384, E=8, k=2, capacity_factor=1.0,
                           bias=SKEW_BIAS),
    "fine_reroute": Workload("cn_fine", T=256, d=256, F=128, E=32, k=6, S=2,
                             gating=SOFTMAX_THEN_TOPK, renormalize=False,
                             capacity_factor=1.0, overflow=1),
    "decode": Workload("cn_dec", T=5, d=256, F=512, E=8, k=2),
    "f32": Workload("cn_f32", T=150, d=72, F=40, E=6, k=2, S=2, dtype="f32",
                    capacity_factor=1.0),
}


@pytest.fixture
def canaries():
    moe.moe_debug_canaries(True)
    yield
    moe.moe_debug_canaries(False)


@pytest.mark.parametrize("case", sorted(CASES))
def test_no_kernel_writes_past_its_region(case, canaries):
    w = CASES[case]
    say(f"[canaries] {case}")
    run = Run(w)
    cfg = config_for(w, bias=run.bias, stream=None)
    ws = moe.Workspace(moe.moe_workspace_size(cfg))
    ws.bind(cfg)
    out = torch.empty((w.T, w.d), dtype=w.torch_dtype, device=DEV)
    moe.moe_forward(run.x, run.Wg, run.W1, run.W3, run.W2, cfg, out, stats=True)
    assert moe.moe_debug_check(cfg) == 0, moe.moe_last_error()
    dout = torch.randn((w.T, w.d), device=DEV).to(w.torch_dtype)
    dl = torch.empty((w.T, w.E), dtype=torch.float32, device=DEV)
    dW = torch.empty((w.d, w.E), dtype=torch.float32, device=DEV)
    db = torch.empty((w.E,), dtype=torch.float32, device=DEV)
    dx = torch.empty((w.T, w.d), dtype=torch.float32, device=DEV)
    moe.moe_router_backward(run.x, run.Wg, dout, cfg, dl, dW, db, dx, aux_coef=0.01,
                            entropy_coef=0.001)
    assert moe.moe_debug_check(cfg) == 0, moe.moe_last_error()
    r = route_buffers(w.T, w.E, w.k)
    moe.moe_route(run.x, run.Wg, cfg, r["logits"], r["idx"], r["w"], r["counts"], r["offsets"],
                  r["perm"], r["slot"], stats=True)
    assert moe.moe_debug_check(cfg) == 0, moe.moe_last_error()
    if w.bias is None:
        moe.moe_route_logits(r["logits"], cfg, r["idx"], r["w"], r["counts"], r["offsets"],
                             r["perm"], r["slot"], stats=True)
        assert moe.moe_debug_check(cfg) == 0, moe.moe_last_error()
        moe.moe_aux_loss(r["logits"], r["counts"], cfg)
        assert moe.moe_debug_check(cfg) == 0, moe.moe_last_error()


def test_overwritten_guard_is_reported(canaries):
    w = CASES["wide_drops"]
    run = Run(w)
    cfg = config_for(w, bias=run.bias, stream=None)
    n = moe.moe_workspace_size(cfg)
    ws = moe.Workspace(n)
    ws.bind(cfg)
    out = torch.empty((w.T, w.d), dtype=w.torch_dtype, device=DEV)
    moe.moe_forward(run.x, run.Wg, run.W1, run.W3, run.W2, cfg, out)
    assert moe.moe_debug_check(cfg) == 0
    # the plan of a bf16 layer ends with the router backward's bf16 W_gate
    # copy (bWt) and its guard: clear one byte of that guard from the host
    start = ws.ptr - ws.buf.data_ptr()
    torch.cuda.synchronize()
    ws.buf[start + n - 1] = 0
    torch.cuda.synchronize()
    assert moe.moe_debug_check(cfg) == 1
    assert "'bWt'" in moe.moe_last_error()

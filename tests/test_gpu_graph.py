"""The forward and the router backward under HIP graph capture.

Without statistics, moe_forward and moe_router_backward enqueue only kernel
launches on cfg->stream (no allocation, no copy, no memset, no host wait),
so a caller can capture them into a graph and replay it.  Each test captures
one call, replays the graph several times with eager library work on the
same buffers in between, and checks every replay bitwise against an eager
call on the same inputs, including after the inputs change in place.
"""
import pytest
import torch

import sparse_mixture_experts_capacity_amd as moe
from gpu_helpers import DEV, Run, say
from workloads import SKEW_BIAS, SOFTMAX_THEN_TOPK, Workload

pytestmark = pytest.mark.gpu

GRAPH_CASES = {
    # one token: the launch-bound decode shape
    "decode_t1": Workload("g_t1", T=1, d=256, F=512, E=8, k=2),
    # several tiles per expert, drops, a shared expert
    "multi_tile_shared": Workload("g_mt", T=600, d=256, F=256, E=8, k=2, S=1,
                                  capacity_factor=1.0, bias=SKEW_BIAS),
    # rerouting pass and fine-grained experts
    "reroute_fine": Workload("g_rr", T=300, d=128, F=128, E=32, k=4,
                             gating=SOFTMAX_THEN_TOPK, renormalize=False,
                             capacity_factor=0.8, overflow=1),
}


def _cfg(w, run, stream):
    cfg = moe.make_config(T=w.T, d_model=w.d, d_ff=w.F, n_experts=w.E, top_k=w.k,
                          n_shared=w.S, gating=w.gating, renormalize=w.renormalize,
                          capacity_factor=w.capacity_factor, dtype=w.dtype,
                          logit_bias=run.bias, stream=stream, overflow=w.overflow)
    ws = moe.Workspace(moe.moe_workspace_size(cfg))
    ws.bind(cfg)
    return cfg, ws


@pytest.mark.parametrize("case", sorted(GRAPH_CASES))
def test_forward_graph_replay(case):
    w = GRAPH_CASES[case]
    say(f"[graph] forward {case}")
    run = Run(w)
    s = torch.cuda.Stream()
    cfg, ws = _cfg(w, run, s)
    out = torch.empty((w.T, w.d), dtype=w.torch_dtype, device=DEV)
    x = run.x.clone()

    def fwd():
        moe.moe_forward(x, run.Wg, run.W1, run.W3, run.W2, cfg, out)

    with torch.cuda.stream(s):
        fwd()
    s.synchronize()
    ref = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fwd()
    for rep in range(3):
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            fwd()                      # eager work on the same workspace between replays
        s.synchronize()
        out.fill_(7.0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16) if w.dtype == "bf16" else out,
                           ref.view(torch.int16) if w.dtype == "bf16" else ref), rep
    # new input values in the same buffer: a replay computes the layer for them
    x.copy_(-run.x)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        fwd()
    s.synchronize()
    ref2 = out.clone()
    assert not torch.equal(ref2, ref)
    out.fill_(7.0)
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(out, ref2)


def test_router_backward_graph_replay():
    w = Workload("g_bw", T=200, d=256, F=256, E=16, k=2, capacity_factor=1.0)
    say("[graph] router backward")
    run = Run(w)
    s = torch.cuda.Stream()
    cfg, ws = _cfg(w, run, s)
    out = torch.empty((w.T, w.d), dtype=w.torch_dtype, device=DEV)
    gen = torch.Generator(device=DEV).manual_seed(3)
    dout = torch.randn((w.T, w.d), generator=gen, device=DEV).to(w.torch_dtype)
    bufs = dict(dl=torch.empty((w.T, w.E), device=DEV), dW=torch.empty((w.d, w.E), device=DEV),
                db=torch.empty((w.E,), device=DEV), dx=torch.empty((w.T, w.d), device=DEV))

    def step():
        moe.moe_forward(run.x, run.Wg, run.W1, run.W3, run.W2, cfg, out)
        moe.moe_router_backward(run.x, run.Wg, dout, cfg, bufs["dl"], bufs["dW"], bufs["db"],
                                bufs["dx"], aux_coef=0.1, entropy_coef=0.05)

    with torch.cuda.stream(s):
        step()
    s.synchronize()
    ref = {k: v.clone() for k, v in bufs.items()}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    for rep in range(3):
        for v in bufs.values():
            v.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for k in bufs:
            assert torch.equal(bufs[k], ref[k]), (k, rep)

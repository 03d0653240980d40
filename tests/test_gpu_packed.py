"""Packed expert weights (moe_weight_layout_t PACKED).

moe_pack_weights must place every element where include/moe.h says, with
zero pad columns; a forward on the packed copies must give the same bits as
the forward on the row-major weights (the layout changes addresses only, not
the arithmetic or its order).  The cases cover every GEMM tile shape (32-row
tiles with 256- and 128-wide weight tiles, 128- and 256-row tiles), widths
that are not multiples of the block widths (padding), shared experts and the
K-split down projection of short batches.
"""
import pytest
import torch

import sparse_mixture_experts_capacity_amd as moe
from gpu_helpers import DEV, Run, config_for, say
from workloads import SKEW_BIAS, SOFTMAX_THEN_TOPK, Workload

pytestmark = pytest.mark.gpu


def reference_pack(W: torch.Tensor, block: int) -> torch.Tensor:
    """[n, K, N] -> flat packed copy by index arithmetic on the host."""
    n, K, N = W.shape
    Np = -(-N // block) * block
    P = torch.zeros((n, K, Np), dtype=W.dtype)
    P[:, :, :N] = W
    # [expert, k block, n block, column in block, k in block]
    return P.view(n, K // 32, 32, Np // block, block).permute(0, 1, 3, 4, 2).reshape(-1)


def packed_copies(run: Run, cfg):
    w13, w2 = moe.moe_packed_weight_bytes(cfg)
    W1p = torch.empty(w13 // 2, dtype=torch.bfloat16, device=DEV)
    W3p = torch.empty(w13 // 2, dtype=torch.bfloat16, device=DEV)
    W2p = torch.empty(w2 // 2, dtype=torch.bfloat16, device=DEV)
    moe.moe_pack_weights(run.W1, run.W3, run.W2, cfg, W1p, W3p, W2p)
    torch.cuda.synchronize()
    return W1p, W3p, W2p


def test_pack_layout_matches_header():
    w = Workload("pack", T=4, d=192, F=320, E=3, k=1, S=2)
    say("[packed] layout of W1, W3 (128-wide blocks) and W2 (256-wide blocks)")
    run = Run(w)
    cfg = config_for(w)
    W1p, W3p, W2p = packed_copies(run, cfg)
    W1, W3, W2 = (t.cpu() for t in (run.W1, run.W3, run.W2))
    for got, ref in ((W1p, reference_pack(W1, 128)), (W3p, reference_pack(W3, 128)),
                     (W2p, reference_pack(W2, 256))):
        assert got.numel() == ref.numel()
        assert torch.equal(got.cpu().view(torch.int16), ref.view(torch.int16))


PACKED_CASES = {
    # one token: 32-row tiles, 256-wide W1/W3 tiles, down projection split
    "decode_t1": Workload("p_t1", T=1, d=256, F=512, E=8, k=2),
    # several hit experts: 128-wide W1/W3 tiles (two per 128-column block)
    "decode_t16_narrow": Workload("p_t16", T=16, d=256, F=384, E=8, k=2),
    # ~150 rows per expert: 256-row tiles; F and d not multiples of the blocks
    "wide_ragged": Workload("p_wide", T=600, d=192, F=320, E=8, k=2, capacity_factor=1.25),
    # ~400 rows per expert: 128-row tiles with the token-row gather, shared
    # experts (their down projection contracts both experts' blocks in one K)
    "long_shared": Workload("p_long", T=1600, d=128, F=320, E=4, k=1, S=2),
    # fine-grained experts, DeepSeek gating, skewed scores with drops
    "fine_drops": Workload("p_fine", T=300, d=256, F=128, E=32, k=6, S=1,
                           gating=SOFTMAX_THEN_TOPK, renormalize=False, capacity_factor=0.8),
    "skew_drops": Workload("p_skew", T=900, d=256, F=384, E=8, k=2, capacity_factor=1.0,
                           bias=SKEW_BIAS),
}


@pytest.mark.parametrize("case", sorted(PACKED_CASES))
def test_forward_packed_equals_row_major(case):
    w = PACKED_CASES[case]
    say(f"[packed] forward {case}")
    run = Run(w)
    out_rm, _ = run.forward(stats=False)
    cfg = moe.make_config(T=w.T, d_model=w.d, d_ff=w.F, n_experts=w.E, top_k=w.k,
                          n_shared=w.S, gating=w.gating, renormalize=w.renormalize,
                          capacity_factor=w.capacity_factor, dtype=w.dtype,
                          logit_bias=run.bias, stream=None, weight_layout=moe.WEIGHTS_PACKED)
    W1p, W3p, W2p = packed_copies(run, cfg)
    ws = moe.Workspace(moe.moe_workspace_size(cfg))
    ws.bind(cfg)
    out = torch.full((w.T, w.d), 7.0, dtype=w.torch_dtype, device=DEV)
    st = moe.moe_forward(run.x, run.Wg, W1p, W3p, W2p, cfg, out, stats=True)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out_rm.view(torch.int16))
    assert st["dropped"] >= 0


def _packed_cfg(w, run, stream=None):
    return moe.make_config(T=w.T, d_model=w.d, d_ff=w.F, n_experts=w.E, top_k=w.k,
                           n_shared=w.S, gating=w.gating, renormalize=w.renormalize,
                           capacity_factor=w.capacity_factor, dtype=w.dtype,
                           logit_bias=run.bias, stream=stream,
                           weight_layout=moe.WEIGHTS_PACKED)


def test_router_backward_after_packed_forward():
    # the backward reads the forward's expert rows: the same bits either way
    w = PACKED_CASES["fine_drops"]
    say("[packed] router backward after a packed forward")
    run = Run(w)
    gen = torch.Generator(device=DEV).manual_seed(5)
    dout = torch.randn((w.T, w.d), generator=gen, device=DEV).to(w.torch_dtype)
    results = []
    for packed in (False, True):
        cfg = _packed_cfg(w, run) if packed else config_for(w, bias=run.bias)
        Ws = packed_copies(run, cfg) if packed else (run.W1, run.W3, run.W2)
        ws = moe.Workspace(moe.moe_workspace_size(cfg))
        ws.bind(cfg)
        out = torch.empty((w.T, w.d), dtype=w.torch_dtype, device=DEV)
        moe.moe_forward(run.x, run.Wg, *Ws, cfg, out)
        bufs = [torch.empty((w.T, w.E), device=DEV), torch.empty((w.d, w.E), device=DEV),
                torch.empty((w.E,), device=DEV), torch.empty((w.T, w.d), device=DEV)]
        moe.moe_router_backward(run.x, run.Wg, dout, cfg, *bufs, aux_coef=0.05, entropy_coef=0.01)
        torch.cuda.synchronize()
        results.append(bufs)
    for a, b in zip(*results):
        assert torch.equal(a, b)


def test_packed_forward_graph_replay():
    w = PACKED_CASES["long_shared"]
    say("[packed] forward captured into a graph")
    run = Run(w)
    s = torch.cuda.Stream()
    cfg = _packed_cfg(w, run, stream=s)
    W1p, W3p, W2p = packed_copies(run, cfg)
    ws = moe.Workspace(moe.moe_workspace_size(cfg))
    ws.bind(cfg)
    out = torch.empty((w.T, w.d), dtype=w.torch_dtype, device=DEV)
    with torch.cuda.stream(s):
        moe.moe_forward(run.x, run.Wg, W1p, W3p, W2p, cfg, out)
    s.synchronize()
    ref = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        moe.moe_forward(run.x, run.Wg, W1p, W3p, W2p, cfg, out)
    for rep in range(3):
        out.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), rep

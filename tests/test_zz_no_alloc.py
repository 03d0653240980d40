"""moe_forward_noalloc: the forward with the library's fixed scratch array
instead of a caller workspace (for callers that cannot allocate).  Through
the C ABI, two calls in a row on one GPU (the second with fewer tokens, so
the array holds the first call's leftovers) must give exactly the bits and
statistics of moe_forward with a fresh workspace."""
import pytest
import torch

import sparse_mixture_experts_capacity_amd as moe
from gpu_helpers import DEV, Run, config_for, say
from workloads import SKEW_BIAS, SOFTMAX_THEN_TOPK, Workload

pytestmark = pytest.mark.gpu

CASES = {
    # Mixtral-shaped experts, capacity drops: 64 tokens, then 8
    "mixtral_like": (Workload("na_mix", T=64, d=1024, F=2048, E=8, k=2, capacity_factor=1.0,
                              bias=SKEW_BIAS), 8),
    # fine-grained experts, shared experts, softmax over all, rerouting:
    # 200 tokens, then 33
    "fine_grained": (Workload("na_fine", T=200, d=512, F=256, E=64, k=6, S=2,
                              gating=SOFTMAX_THEN_TOPK, renormalize=False,
                              capacity_factor=1.0, overflow=1), 33),
}


def _pair(run, T, packed=False):
    w = run.w
    cfg = config_for(w, T=T, bias=run.bias, stream=None, packed=packed)
    W = run.packed_weights(cfg) if packed else (run.W1, run.W3, run.W2)
    ws = moe.Workspace(moe.moe_workspace_size(cfg))
    ws.bind(cfg)
    ref = torch.empty((T, w.d), dtype=w.torch_dtype, device=DEV)
    st_ref = moe.moe_forward(run.x[:T], run.Wg, *W, cfg, ref, stats=True)
    del ws
    cfg_na = config_for(w, T=T, bias=run.bias, stream=None, packed=packed)
    out = torch.full((T, w.d), float("nan"), dtype=w.torch_dtype, device=DEV)
    st = moe.moe_forward_noalloc(run.x[:T], run.Wg, *W, cfg_na, out, stats=True)
    torch.cuda.synchronize()
    return ref, st_ref, out, st


@pytest.mark.parametrize("case", sorted(CASES))
def test_noalloc_matches_forward(case):
    w, T2 = CASES[case]
    run = Run(w)
    for T in (w.T, T2):
        for packed in (False, True):
            say(f"[noalloc] {case}: T={T} packed={packed}")
            ref, st_ref, out, st = _pair(run, T, packed)
            assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
            for key in ("capacity", "dropped", "overflowed", "rerouted", "rounds"):
                assert st[key] == st_ref[key], key
            assert (st["counts"] == st_ref["counts"]).all()
            assert (st["kept"] == st_ref["kept"]).all()
            for key in ("aux_loss", "entropy_load", "entropy_token"):
                assert st[key] == st_ref[key], key


def test_noalloc_without_stats_and_empty():
    w, _ = CASES["mixtral_like"]
    run = Run(w)
    cfg = config_for(w, bias=run.bias, stream=None)
    out = torch.empty((w.T, w.d), dtype=w.torch_dtype, device=DEV)
    moe.moe_forward_noalloc(run.x, run.Wg, run.W1, run.W3, run.W2, cfg, out)
    torch.cuda.synchronize()
    ref, _, _, _ = _pair(run, w.T)
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    empty = config_for(w, T=0, bias=run.bias, stream=None)
    st = moe.moe_forward_noalloc(run.x[:0], run.Wg, run.W1, run.W3, run.W2, empty,
                                 out[:0], stats=True)
    assert st["dropped"] == 0 and st["aux_loss"] == 0.0

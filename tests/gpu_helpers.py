"""Shared plumbing of the GPU parity tests: run the HIP library through its
C ABI on seeded inputs and run the oracle on the same bytes."""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

import oracle.oracle as O
import sparse_mixture_experts_capacity_amd as moe
from workloads import Workload, make_inputs

DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def config_for(w: Workload, T=None, path=moe.PATH_AUTO, bias=None, stream=None, packed=False):
    return moe.make_config(
        T=w.T if T is None else T, d_model=w.d, d_ff=w.F, n_experts=w.E,
        top_k=w.k, n_shared=w.S, gating=w.gating, renormalize=w.renormalize,
        capacity_factor=w.capacity_factor, dtype=w.dtype, ffn_path=path,
        logit_bias=bias, stream=stream, overflow=w.overflow,
        weight_layout=moe.WEIGHTS_PACKED if packed else moe.WEIGHTS_ROW_MAJOR)


def shape_of(w: Workload, T=None) -> O.LayerShape:
    return O.LayerShape(T=w.T if T is None else T, d=w.d, F=w.F, E=w.E, k=w.k,
                        S=w.S, gating=w.gating, renormalize=w.renormalize,
                        capacity_factor=w.capacity_factor, overflow=w.overflow)


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


class Run:
    """Inputs of one workload on the GPU plus host copies for the oracle."""

    def __init__(self, w: Workload, seed=0, gen_device="cpu"):
        self.w = w
        t0 = time.time()
        inp = make_inputs(w, seed=seed, device=gen_device)
        self.x = inp.x.to(DEV)
        self.Wg = inp.W_gate.to(DEV)
        self.W1 = inp.W1.to(DEV)
        self.W3 = inp.W3.to(DEV)
        self.W2 = inp.W2.to(DEV)
        self.bias = inp.bias.to(DEV) if inp.bias is not None else None
        # host copies (bf16/fp32 as stored); widened per expert on demand
        self.hx = inp.x.cpu()
        self.hWg = inp.W_gate.cpu()
        self.hbias = inp.bias.cpu() if inp.bias is not None else None
        self._hW = None
        self._packed = None
        say(f"  inputs {w.name} T={w.T} d={w.d} F={w.F} E={w.E} k={w.k} S={w.S} "
            f"on {gen_device}: {time.time() - t0:.1f}s")

    def host_weights(self):
        if self._hW is None:
            self._hW = (self.W1.cpu(), self.W3.cpu(), self.W2.cpu())
        return self._hW

    def expert(self, e):
        W1, W3, W2 = self.host_weights()
        return to64(W1[e]), to64(W3[e]), to64(W2[e])

    def packed_weights(self, cfg):
        """Packed copies of W1, W3, W2 (made once, as a server would)."""
        if self._packed is None:
            w13, w2 = moe.moe_packed_weight_bytes(cfg)
            self._packed = tuple(torch.empty(n // 2, dtype=torch.bfloat16, device=DEV)
                                 for n in (w13, w13, w2))
            moe.moe_pack_weights(self.W1, self.W3, self.W2, cfg, *self._packed)
            torch.cuda.synchronize()
        return self._packed

    def forward(self, path=moe.PATH_AUTO, stats=True, T=None, packed=False):
        w = self.w
        T = w.T if T is None else T
        cfg = config_for(w, T=T, path=path, bias=self.bias, stream=None, packed=packed)
        W = self.packed_weights(cfg) if packed else (self.W1, self.W3, self.W2)
        ws = moe.Workspace(moe.moe_workspace_size(cfg))
        ws.bind(cfg)
        out = torch.empty((T, w.d), dtype=w.torch_dtype, device=DEV)
        st = moe.moe_forward(self.x[:T], self.Wg, *W, cfg, out, stats=stats)
        torch.cuda.synchronize()
        return out, st

    def route(self, T=None):
        w = self.w
        T = w.T if T is None else T
        cfg = config_for(w, T=T, bias=self.bias, stream=None)
        ws = moe.Workspace(moe.moe_workspace_size(cfg))
        ws.bind(cfg)
        r = route_buffers(T, w.E, w.k)
        st = moe.moe_route(self.x[:T], self.Wg, cfg, r["logits"], r["idx"], r["w"],
                           r["counts"], r["offsets"], r["perm"], r["slot"],
                           stats=True)
        torch.cuda.synchronize()
        return {k: v.cpu() for k, v in r.items()}, st

    def oracle(self, T=None, tokens=None):
        w = self.w
        T = w.T if T is None else T
        return O.forward(to64(self.hx[:T]), shape_of(w, T), self.expert,
                         W_gate=to64(self.hWg),
                         bias=None if self.hbias is None else to64(self.hbias),
                         tokens=tokens)


def route_buffers(T, E, k):
    return dict(
        logits=torch.empty((T, E), dtype=torch.float32, device=DEV),
        idx=torch.full((T, k), -7, dtype=torch.int32, device=DEV),
        w=torch.empty((T, k), dtype=torch.float32, device=DEV),
        counts=torch.full((E,), -7, dtype=torch.int32, device=DEV),
        offsets=torch.full((E + 1,), -7, dtype=torch.int32, device=DEV),
        perm=torch.full((T * k,), -7, dtype=torch.int32, device=DEV),
        slot=torch.full((T * k,), -7, dtype=torch.int32, device=DEV),
    )


def full_order_margin(logits: np.ndarray) -> np.ndarray:
    """Per token, the smallest gap between neighbours of all its sorted
    scores: rerouting reads the whole order, not only the top k + 1."""
    if logits.shape[0] == 0 or logits.shape[1] < 2:
        return np.full(logits.shape[0], np.inf)
    return np.min(np.diff(np.sort(logits, axis=1), axis=1), axis=1)


def near_tie_tokens(gpu_logits: np.ndarray, ref: dict, floor=1e-6, full_order=False):
    """Tokens whose routing decision margin is within the fp32-vs-fp64 logit
    error (or 1e-6): their selection is allowed to differ.  With full_order
    the margin covers every score of the token (rerouting)."""
    err = float(np.max(np.abs(gpu_logits - ref["logits"]))) if gpu_logits.size else 0.0
    thr = max(floor, 4.0 * err)
    margin = full_order_margin(ref["logits"]) if full_order else ref["margin"]
    return np.nonzero(margin < thr)[0], err, thr


def comparable_tokens(w: Workload, ref: dict, ties: np.ndarray, T: int):
    """Tokens whose output is comparable: all but the near ties, and, when
    some assignments overflowed, only tokens before the first near tie
    (a flipped choice shifts every later rank of that expert)."""
    ok = np.ones(T, dtype=bool)
    ok[ties] = False
    if len(ties) and ref["dispatch"]["overflowed"] > 0:
        ok[int(ties.min()):] = False
    return ok


def rel_max_err(got: np.ndarray, ref: np.ndarray):
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    return err, rms


def tol_for(w: Workload):
    return 1e-5 if w.dtype == "f32" else 2e-2


def output_within_tolerance(got: np.ndarray, ref: np.ndarray, w: Workload):
    """Element-wise |got - ref| <= tol * RMS(ref) + fmt * |ref|, with RMS(ref)
    over the rows that are not identically zero (those must match exactly).

    tol is 2e-2 (bf16 layers) or 1e-5 (fp32 layer).  fmt is the largest
    relative error of rounding one value to the output format to nearest-even:
    2^-8 for bf16 (8 significant bits), 2^-24 for fp32.  Every bf16 result
    carries that rounding whatever the arithmetic before it, so it is allowed
    on top of the stated bound.  Returns (ok, max|d| / RMS, worst excess)."""
    if ref.size == 0:
        return True, 0.0, 0.0
    # Rows the layer leaves at exactly zero (every choice dropped, no shared
    # expert) must be exactly zero; RMS(ref) is taken over the other rows, so
    # that a mostly-dropped batch is not held to the scale of its zeros.
    if ref.ndim == 2:
        live = np.any(ref != 0.0, axis=1)
        if not np.all(got[~live] == 0.0):
            return False, float("inf"), float("inf")
        if not live.any():
            return True, 0.0, 0.0
        got, ref = got[live], ref[live]
    rms = float(np.sqrt(np.mean(ref ** 2)))
    fmt = 2.0 ** -24 if w.dtype == "f32" else 2.0 ** -8
    bound = tol_for(w) * rms + fmt * np.abs(ref)
    diff = np.abs(got - ref)
    excess = float(np.max(diff - bound))
    return excess <= 0.0, float(np.max(diff)) / max(rms, 1e-300), excess

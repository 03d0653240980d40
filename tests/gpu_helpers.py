"""Shared plumbing of the GPU parity tests: run the HIP library through its
C ABI on seeded inputs and run the oracle on the same bytes."""
from __future__ import annotations

import json
import os
import sys
import time

import numpy as np
import torch

import oracle.oracle as O
import sparse_mixture_experts_capacity_amd as moe
from workloads import Workload, make_inputs

DEV = "cuda"
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def config_for(w: Workload, T=None, path=moe.PATH_AUTO, bias=None, stream=None, packed=False,
               out_fp32=False):
    return moe.make_config(
        T=w.T if T is None else T, d_model=w.d, d_ff=w.F, n_experts=w.E,
        top_k=w.k, n_shared=w.S, gating=w.gating, renormalize=w.renormalize,
        capacity_factor=w.capacity_factor, dtype=w.dtype, ffn_path=path,
        logit_bias=bias, stream=stream, overflow=w.overflow,
        weight_layout=moe.WEIGHTS_PACKED if packed else moe.WEIGHTS_ROW_MAJOR,
        out_fp32=out_fp32)


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

    def forward(self, path=moe.PATH_AUTO, stats=True, T=None, packed=False, out_fp32=False):
        w = self.w
        T = w.T if T is None else T
        cfg = config_for(w, T=T, path=path, bias=self.bias, stream=None, packed=packed,
                         out_fp32=out_fp32)
        W = self.packed_weights(cfg) if packed else (self.W1, self.W3, self.W2)
        ws = moe.Workspace(moe.moe_workspace_size(cfg))
        ws.bind(cfg)
        out = torch.empty((T, w.d), dtype=torch.float32 if out_fp32 else w.torch_dtype,
                          device=DEV)
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

    def oracle(self, T=None, tokens=None, logits=None):
        """The oracle on these inputs: from fp64 router scores of x, W_gate and
        the bias, or, given ``logits`` (fp64 [T, E], e.g. the GPU's fp32
        scores widened exactly), from those scores."""
        w = self.w
        T = w.T if T is None else T
        if logits is not None:
            return O.forward(to64(self.hx[:T]), shape_of(w, T), self.expert,
                             logits=logits, tokens=tokens)
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
    error (or 1e-6): in the independent-scores check of the router, their
    selection is allowed to differ.  With full_order the margin covers every
    score of the token (rerouting)."""
    err = float(np.max(np.abs(gpu_logits - ref["logits"]))) if gpu_logits.size else 0.0
    thr = max(floor, 4.0 * err)
    margin = full_order_margin(ref["logits"]) if full_order else ref["margin"]
    return np.nonzero(margin < thr)[0], err, thr


def tol_for(w: Workload):
    """The output bound as a multiple of RMS(ref): 2e-2 for bf16 layers, 1e-5
    for the fp32 layer."""
    return 1e-5 if w.dtype == "f32" else 2e-2


def rne_bf16(a: np.ndarray) -> np.ndarray:
    """fp64 values rounded to bf16 (nearest, ties to even), widened back."""
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).to(torch.float64).numpy()


def record(entry: dict) -> None:
    """Append one parity result to parity_ratios.jsonl (the per-workload
    record of max|d| / RMS(ref)) in $MOE_TEST_RECORDS, by default
    test_records/ at the repository root."""
    d = os.environ.get("MOE_TEST_RECORDS") or os.path.join(ROOT, "test_records")
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "parity_ratios.jsonl"), "a") as f:
        f.write(json.dumps(entry) + "\n")


# Named synthetic cases whose outputs are mostly exact zeros (nearly every
# assignment dropped, no shared expert): RMS(ref) is taken over the rows that
# are not identically zero, and those zero rows must be exactly zero.
LIVE_ROW_RMS_CASES = {"bf16_one_slot"}


def check_layer(run: Run, label: str, path=moe.PATH_AUTO, packed=False, tokens=None,
                live_row_rms=False, also_row_major=False, per_gate_mass=False):
    """One layer on the GPU against the oracle, with the strict output bound.

    * The oracle runs on the GPU's own fp32 router scores (widened exactly),
      so routing, gates and dispatch are the same decisions on both sides
      and no token is excluded.  The scores themselves are checked against
      fp64 in the router tests.
    * Routing counts, kept rows, drops and the overflow counts must equal the
      oracle's exactly; the statistics within 1e-5 relative.
    * The layer is run with fp32 output (cfg.out_fp32) and with its own
      output dtype.  A bf16 output must be exactly the fp32 output rounded to
      nearest-even, bit for bit: the final store is the only difference.
    * Bound: max|out_fp32 - ref| <= tol * RMS(ref), RMS over every compared
      row, tol = 2e-2 (bf16 layers) or 1e-5 (fp32).  The ratio of the
      delivered bf16 output, and the floor that rounding the exact result to
      bf16 alone sets (max|RNE(ref) - ref| / RMS(ref)), are reported beside
      it.
    ``tokens`` limits the compared rows (routing always covers every token).
    ``per_gate_mass`` (routed experts only, no drops): every row of ref and
    of the outputs is divided by the token's summed gate weights before the
    comparison, so the bound applies to the gate-weighted mean of the
    token's expert rows; the output of softmax-over-all gates without
    renormalisation is otherwise dominated by the few tokens with the most
    gate mass.  The plain ratio is recorded too.
    Returns the recorded entry."""
    w = run.w
    out_f32, st = run.forward(path=path, packed=packed, out_fp32=True)
    out, _ = run.forward(path=path, packed=packed, stats=False)
    if w.dtype == "bf16":
        assert torch.equal(out.view(torch.int16), out_f32.to(torch.bfloat16).view(torch.int16)), \
            "bf16 output is not the RNE rounding of the fp32 output"
    else:
        assert torch.equal(out, out_f32)
    if also_row_major and packed:
        out_rm, _ = run.forward(path=path, packed=False, stats=False)
        assert torch.equal(out.view(torch.int16), out_rm.view(torch.int16)), \
            "packed and row-major weights give other bits"
        del out_rm
    g_route, _ = run.route()
    L = g_route["logits"].numpy().astype(np.float64)
    ref = run.oracle(logits=L, tokens=tokens)
    D = ref["dispatch"]
    assert np.array_equal(g_route["idx"].numpy().astype(np.int64), ref["sel"])
    assert np.array_equal(st["counts"], D["counts"])
    assert np.array_equal(st["kept"], D["kept"])
    assert st["capacity"] == D["capacity"] and st["dropped"] == D["dropped"]
    for key in ("overflowed", "rerouted", "rounds"):
        assert st[key] == D[key], key
    for key in ("aux_loss", "aux_loss_kept", "overflow_rate", "entropy_load", "entropy_token"):
        r = ref["stats"][key]
        assert abs(st[key] - r) <= 1e-5 * max(abs(r), 1e-3), (key, st[key], r)

    rows = np.arange(w.T) if tokens is None else np.asarray(sorted(set(tokens)), dtype=np.int64)
    r = ref["out"][rows]
    g32 = to64(out_f32)[rows]
    g = to64(out)[rows]
    assert np.all(np.isfinite(g32)) and np.all(np.isfinite(g))
    plain = None
    if per_gate_mass:
        assert w.S == 0 and D["dropped"] == 0
        mass = ref["w"][rows].sum(axis=1)[:, None]
        rms0 = float(np.sqrt(np.mean(r ** 2)))
        plain = float(np.max(np.abs(g32 - r))) / rms0
        r, g32, g = r / mass, g32 / mass, g / mass
    if live_row_rms:
        live = np.any(r != 0.0, axis=1)
        assert np.all(g32[~live] == 0.0) and np.all(g[~live] == 0.0)
        plain = float(np.max(np.abs(g32 - r))) / float(np.sqrt(np.mean(r ** 2)))
        r, g32, g = r[live], g32[live], g[live]
    rms = float(np.sqrt(np.mean(r ** 2))) if r.size else 0.0
    tol = tol_for(w)
    if r.size == 0:
        ratio32 = ratio = floor = 0.0
    else:
        ratio32 = float(np.max(np.abs(g32 - r))) / rms
        ratio = float(np.max(np.abs(g - r))) / rms
        floor = float(np.max(np.abs(rne_bf16(r) - r))) / rms if w.dtype == "bf16" else 0.0
    entry = dict(label=label, workload=w.name, T=w.T, d=w.d, F=w.F, E=w.E, k=w.k, S=w.S,
                 overflow=w.overflow, dtype=w.dtype, packed=bool(packed), path=int(path),
                 rows_compared=int(len(rows)), elements=int(r.size), rms_ref=rms,
                 ratio_fp32_out=ratio32, ratio_out=ratio, bf16_rounding_floor=floor,
                 tol=tol, dropped=int(D["dropped"]), rerouted=int(D["rerouted"]),
                 rms_over="live rows" if live_row_rms else "all compared rows",
                 per_gate_mass=bool(per_gate_mass), ratio_fp32_out_plain=plain)
    record(entry)
    say(f"  {label}: {len(rows)} rows, RMS(ref) {rms:.3e}: max|d|/RMS fp32-out {ratio32:.3e} "
        f"(bound {tol:g}), {w.dtype} out {ratio:.3e}, rounding floor {floor:.3e}; "
        f"dropped {D['dropped']} rerouted {D['rerouted']}")
    assert ratio32 <= tol, f"{label}: max|d| = {ratio32:.3e} RMS(ref) exceeds {tol:g}"
    return entry

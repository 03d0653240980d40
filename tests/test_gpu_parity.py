"""GPU parity of the HIP library against the fp64 oracle, through the C ABI.

* routing / dispatch / statistics from the same fp32 logits: bit-exact
  indices, counts, offsets, permutation and slots (moe_route_logits);
* router GEMM scores against fp64, and selections away from near ties;
* full layer outputs, oracle fed the GPU's own fp32 scores: max|d| <= 2e-2 *
  RMS(ref) for bf16 and 1e-5 * RMS(ref) for fp32 over every compared row, on
  the layer's fp32 output, with the bf16 output exactly its RNE rounding; at
  sizes spanning several tiles with ragged tails, and at the full workload
  sizes on every token (the skewed 16384-token layers on 4096 tokens that
  cover every drop and reroute class);
* determinism and the empty call.
"""
import math

import numpy as np
import pytest
import torch

import oracle.oracle as O
import sparse_mixture_experts_capacity_amd as moe
from gpu_helpers import (DEV, LIVE_ROW_RMS_CASES, Run, check_layer, config_for,
                         near_tie_tokens, route_buffers, say, to64)
from workloads import PRESETS, SKEW_BIAS, SOFTMAX_THEN_TOPK, Workload, normal, random_logits

pytestmark = pytest.mark.gpu


# --------------------------------------------------------------------------
# routing from the same fp32 logits: bit-exact
# --------------------------------------------------------------------------
def _logits_case(name):
    if name == "tiny":
        w = PRESETS["tiny_f32"]
        r = Run(w)  # CPU-generated; logits from the oracle's own router
        L = torch.tensor(O.router_logits(to64(r.hx), to64(r.hWg)), dtype=torch.float32)
        return w, L
    if name == "prefill":
        w = PRESETS["mixtral_prefill"]
        return w, random_logits(w.T, w.E, seed=1)
    if name == "skew_cf1.0":
        w = PRESETS["skew_cf1.0"]
        return w, random_logits(w.T, w.E, seed=2) + torch.tensor(SKEW_BIAS)
    if name == "skew_cf1.5":
        w = PRESETS["skew_cf1.5"]
        return w, random_logits(w.T, w.E, seed=3) + torch.tensor(SKEW_BIAS)
    if name == "deepseek":
        w = PRESETS["deepseek"]
        return w, random_logits(w.T, w.E, seed=4)
    if name == "ties_signed_zero":
        w = Workload("ties", T=3000, d=64, F=64, E=8, k=2, capacity_factor=1.1)
        L = torch.round(random_logits(w.T, w.E, seed=5))
        L[L == 0] = 0.0
        L[::3, 2] = -0.0
        L[::5, 5] = 0.0
        return w, L
    if name == "all_equal":
        w = Workload("all_equal", T=1500, d=64, F=64, E=16, k=4, capacity_factor=1.0)
        L = torch.zeros(w.T, w.E)
        L[torch.rand(w.T, w.E, generator=torch.Generator().manual_seed(6)) < 0.5] = -0.0
        return w, L
    if name == "E256_k8":
        w = Workload("E256", T=700, d=64, F=64, E=256, k=8, capacity_factor=1.0)
        return w, random_logits(w.T, w.E, seed=7)
    if name == "k_equals_E":
        w = Workload("kE", T=100, d=64, F=64, E=8, k=8)
        return w, random_logits(w.T, w.E, seed=8)
    if name == "E1":
        w = Workload("E1", T=50, d=64, F=64, E=1, k=1, capacity_factor=0.5)
        return w, random_logits(w.T, w.E, seed=9)
    if name == "T1":
        w = Workload("T1", T=1, d=64, F=64, E=8, k=2)
        return w, random_logits(w.T, w.E, seed=10)
    if name == "tiny_capacity":
        w = Workload("tinycap", T=5000, d=64, F=64, E=8, k=2, capacity_factor=0.01)
        return w, random_logits(w.T, w.E, seed=11) * 3
    if name == "nan_scores":
        # NaN scores rank as -infinity; every row keeps at least one number
        w = Workload("nan", T=500, d=64, F=64, E=8, k=2, capacity_factor=1.0)
        L = random_logits(w.T, w.E, seed=13)
        g = torch.Generator().manual_seed(14)
        mask = torch.rand(w.T, w.E, generator=g) < 0.3
        mask[:, 0] = False
        mask[::7, 1:] = True      # rows with a single number
        L[mask] = float("nan")
        return w, L
    if name == "deepseek_cf1.0":
        # 160 fine-grained experts at capacity factor 1: spare experts abound
        w = PRESETS["deepseek"].with_(capacity_factor=1.0)
        return w, random_logits(w.T, w.E, seed=16) * 2
    if name == "short_batch_skew":
        # T <= 128: the fused one-workgroup routing, unless overflow is rerouted
        w = Workload("short_skew", T=100, d=64, F=64, E=8, k=2, capacity_factor=0.75)
        return w, random_logits(w.T, w.E, seed=15) + torch.tensor(SKEW_BIAS)
    if name == "pair_skew":
        # experts 0 and 1 are every token's favourites: late tokens overflow on
        # both choices, and a spare expert with room must not take one token
        # twice
        w = Workload("pair_skew", T=3000, d=64, F=64, E=8, k=2, capacity_factor=1.25)
        L = random_logits(w.T, w.E, seed=18)
        L[:, :2] += 3.0
        return w, L
    if name == "triple_skew_k4":
        w = Workload("triple_skew", T=2000, d=64, F=64, E=16, k=4, capacity_factor=1.0)
        L = random_logits(w.T, w.E, seed=19)
        L[:, :3] += 3.0
        return w, L
    if name == "deepseek_renorm_k1":
        w = Workload("dsr", T=777, d=64, F=64, E=64, k=1, gating=SOFTMAX_THEN_TOPK,
                     renormalize=True, capacity_factor=1.25)
        return w, random_logits(w.T, w.E, seed=12)
    raise KeyError(name)


LOGIT_CASES = ["tiny", "prefill", "skew_cf1.0", "skew_cf1.5", "deepseek",
               "ties_signed_zero", "all_equal", "E256_k8", "k_equals_E", "E1", "T1",
               "tiny_capacity", "deepseek_renorm_k1", "nan_scores"]


REROUTE_CASES = ["tiny", "prefill", "skew_cf1.0", "deepseek", "ties_signed_zero", "all_equal",
                 "E256_k8", "k_equals_E", "E1", "T1", "tiny_capacity", "nan_scores",
                 "short_batch_skew", "deepseek_cf1.0", "pair_skew", "triple_skew_k4"]
SEQUENTIAL_CASES = ["skew_cf1.0", "deepseek", "tiny_capacity", "short_batch_skew", "T1"]


@pytest.mark.parametrize("case", LOGIT_CASES + ["short_batch_skew"])
def test_route_logits_bit_exact(case):
    _route_logits_case(case, O.OVERFLOW_DROP)


@pytest.mark.parametrize("case", REROUTE_CASES)
def test_route_logits_reroute_bit_exact(case):
    _route_logits_case(case, O.OVERFLOW_REROUTE)


@pytest.mark.parametrize("case", SEQUENTIAL_CASES)
def test_route_logits_sequential_bit_exact(case):
    _route_logits_case(case, O.OVERFLOW_SEQUENTIAL)


def _route_logits_case(case, policy):
    say(f"[route_logits] {case} overflow policy {policy}")
    w, L = _logits_case(case)
    _check_route_logits(w.with_(overflow=policy), L, policy)


def _check_route_logits(w, L, policy):
    T, E, k = w.T, w.E, w.k
    # oracle on the same fp32 values, widened exactly (a NaN score ranks as
    # -infinity in the library; the oracle, which takes numbers only, gets -1e30)
    L64 = L.to(torch.float64).numpy()
    L64 = np.where(np.isnan(L64), -1e30, L64)
    sel, margin = O.topk_select(L64, k)
    gates = O.gate_weights(L64, sel, w.gating, w.renormalize)
    C = O.capacity(T, k, E, w.capacity_factor)
    D = O.dispatch_policy(sel, L64, E, C, policy)
    st_ref = O.routing_stats(D["counts"], D["kept"], O.softmax_all(L64), T, k, E)

    cfg = config_for(w, stream=None)
    ws = moe.Workspace(moe.moe_workspace_size(cfg))
    ws.bind(cfg)
    r = route_buffers(T, E, k)
    Ld = L.to(DEV).contiguous()
    st = moe.moe_route_logits(Ld, cfg, r["idx"], r["w"], r["counts"], r["offsets"],
                               r["perm"], r["slot"], stats=True)
    torch.cuda.synchronize()
    g = {n: v.cpu().numpy() for n, v in r.items()}

    assert np.array_equal(g["idx"].astype(np.int64), sel), "top-k indices differ"
    assert np.array_equal(g["counts"].astype(np.int64), D["counts"])
    assert np.array_equal(g["offsets"].astype(np.int64), D["offsets"])
    total = int(D["offsets"][-1])
    assert np.array_equal(g["perm"][:total].astype(np.int64), D["perm"])
    assert np.all(g["perm"][total:] == -1)
    assert np.array_equal(g["slot"].astype(np.int64), D["slot"])
    # gates: fp32 exp vs fp64
    assert np.max(np.abs(g["w"] - gates)) <= 2e-6 * max(1.0, float(np.max(gates)))
    # statistics
    assert st["capacity"] == C and st["dropped"] == D["dropped"]
    assert np.array_equal(st["counts"], D["counts"])
    assert np.array_equal(st["kept"], D["kept"])
    assert (st["overflowed"], st["rerouted"], st["rounds"]) == \
        (D["overflowed"], D["rerouted"], D["rounds"])
    for key in ("aux_loss", "aux_loss_kept", "overflow_rate", "entropy_load",
                "entropy_token"):
        ref = st_ref[key]
        assert abs(st[key] - ref) <= 1e-5 * max(abs(ref), 1e-3), (key, st[key], ref)
    say(f"  ok: C={C} overflowed={D['overflowed']} rerouted={D['rerouted']} "
        f"dropped={D['dropped']} rounds={D['rounds']} aux={st['aux_loss']:.6f} "
        f"min margin={float(margin.min()) if T else 0:.3g}")


# seeded random configurations: expert counts from 1 to 256, k up to 8,
# batch sizes on both sides of the one-workgroup routing limit, capacity
# factors from 0.3 to unlimited, both gating orders, every overflow policy,
# and scores rounded to halves in some cases so that many ties occur
def _sweep_case(i):
    rng = np.random.default_rng(1000 + i)
    E = int(rng.choice([1, 2, 3, 5, 8, 13, 16, 32, 64, 100, 160, 256]))
    k = int(rng.integers(1, min(E, 8) + 1))
    T = int(rng.choice([1, 3, 17, 64, 100, 129, 500, 1000, 2500, 4097]))
    cf = float(rng.choice([0.0, 0.3, 0.75, 1.0, 1.25, 2.0]))
    gating = int(rng.integers(0, 2))
    renorm = bool(rng.integers(0, 2))
    policy = int(rng.choice([O.OVERFLOW_DROP, O.OVERFLOW_REROUTE, O.OVERFLOW_SEQUENTIAL]))
    w = Workload(f"sweep{i}", T=T, d=64, F=64, E=E, k=k, gating=gating, renormalize=renorm,
                 capacity_factor=cf, overflow=policy)
    L = random_logits(T, E, seed=2000 + i, scale=float(rng.choice([0.5, 1.0, 4.0])))
    if rng.random() < 0.3:
        L = torch.round(L * 2.0) / 2.0
    return w, L, policy


@pytest.mark.parametrize("i", range(24))
def test_route_logits_random_sweep(i):
    w, L, policy = _sweep_case(i)
    say(f"[sweep {i}] T={w.T} E={w.E} k={w.k} cf={w.capacity_factor} gating={w.gating} "
        f"renorm={w.renormalize} policy={policy}")
    _check_route_logits(w, L, policy)


# Dispatch at the edges of its batching: the chunk pass ranks 1024
# assignments per workgroup and the scan reads each expert's chunk totals 16
# at a time (16, 17 and 32 chunks below); the slot offsets are scanned by one
# wavefront with 1, 2 or 4 experts per lane (E = 64, 65, 200).
DISPATCH_EDGE_CASES = {
    "chunks16_E64": Workload("de16", T=8192, d=64, F=64, E=64, k=2, capacity_factor=1.0),
    "chunks17_E65": Workload("de17", T=8193, d=64, F=64, E=65, k=2, capacity_factor=1.0,
                             gating=SOFTMAX_THEN_TOPK, renormalize=False),
    "chunks17_E65_reroute": Workload("de17r", T=8193, d=64, F=64, E=65, k=2,
                                     capacity_factor=1.0, overflow=O.OVERFLOW_REROUTE),
    "chunks32_E200": Workload("de32", T=4096, d=64, F=64, E=200, k=8, capacity_factor=0.9),
}


@pytest.mark.parametrize("case", sorted(DISPATCH_EDGE_CASES))
def test_dispatch_batch_edges(case):
    w = DISPATCH_EDGE_CASES[case]
    say(f"[dispatch edges] {case}: T*k = {w.T * w.k}, E = {w.E}")
    _check_route_logits(w, random_logits(w.T, w.E, seed=17), w.overflow)


# seeded random bf16 layers: every output element against the oracle
# within the bf16 bound, and the packed weights giving the same bits
def _forward_sweep_case(i):
    rng = np.random.default_rng(3000 + i)
    E = int(rng.choice([1, 2, 4, 8, 16, 32, 64]))
    k = int(rng.integers(1, min(E, 6) + 1))
    T = int(rng.choice([1, 5, 40, 130, 333, 700]))
    d = int(rng.choice([64, 128, 192, 256]))
    F = int(rng.choice([64, 128, 192, 320]))
    S = int(rng.choice([0, 0, 1, 2]))
    cf = float(rng.choice([0.0, 0.5, 1.0, 1.25]))
    gating = int(rng.integers(0, 2))
    policy = int(rng.choice([O.OVERFLOW_DROP, O.OVERFLOW_REROUTE, O.OVERFLOW_SEQUENTIAL]))
    bias = tuple(float(v) for v in rng.normal(0, 1, E)) if rng.random() < 0.3 else None
    return Workload(f"fsweep{i}", T=T, d=d, F=F, E=E, k=k, S=S, gating=gating,
                    renormalize=bool(rng.integers(0, 2)), capacity_factor=cf, overflow=policy,
                    bias=bias)


@pytest.mark.parametrize("i", range(12))
def test_forward_random_sweep(i):
    w = _forward_sweep_case(i)
    say(f"[forward sweep {i}] T={w.T} d={w.d} F={w.F} E={w.E} k={w.k} S={w.S} "
        f"cf={w.capacity_factor} gating={w.gating} policy={w.overflow} bias={w.bias is not None}")
    run = Run(w)
    check_layer(run, f"sweep{i}", packed=True, also_row_major=True)


def test_aux_loss_entry_point():
    say("[aux_loss] skew logits")
    w, L = _logits_case("skew_cf1.0")
    L64 = L.to(torch.float64).numpy()
    sel, _ = O.topk_select(L64, w.k)
    D = O.dispatch(sel, w.E, O.capacity(w.T, w.k, w.E, w.capacity_factor))
    ref = O.routing_stats(D["counts"], D["kept"], O.softmax_all(L64), w.T, w.k, w.E)
    cfg = config_for(w, stream=None)
    ws = moe.Workspace(moe.moe_workspace_size(cfg))
    ws.bind(cfg)
    counts = torch.tensor(D["counts"], dtype=torch.int32, device=DEV)
    aux = moe.moe_aux_loss(L.to(DEV), counts, cfg)
    assert abs(aux - ref["aux_loss"]) <= 1e-5 * ref["aux_loss"]
    assert aux > 1.2   # skew raises it above the balanced value 1


# --------------------------------------------------------------------------
# router GEMM (moe_route): scores against fp64, selections off near ties
# --------------------------------------------------------------------------
ROUTE_CASES = {
    "tiny_f32": PRESETS["tiny_f32"],
    "bf16_E8": Workload("bf16_E8", T=700, d=256, F=64, E=8, k=2, capacity_factor=1.25),
    "bf16_skew": Workload("bf16_skew", T=900, d=512, F=64, E=8, k=2, capacity_factor=1.0,
                          bias=SKEW_BIAS),
    "bf16_E160": Workload("bf16_E160", T=300, d=512, F=64, E=160, k=6,
                          gating=SOFTMAX_THEN_TOPK, renormalize=False),
    "f32_E40_ragged_d": Workload("f32_E40", T=77, d=100, F=30, E=40, k=3, dtype="f32",
                                 capacity_factor=1.0),
    # short batches (one routing workgroup), router scores in K parts, with
    # and without a score bias
    "bf16_fused_T1": Workload("bf16_f1", T=1, d=1024, F=64, E=8, k=2),
    "bf16_fused_T3_E16": Workload("bf16_f3", T=3, d=384, F=64, E=16, k=4,
                                  gating=SOFTMAX_THEN_TOPK, renormalize=False),
    "bf16_fused_T128_bias": Workload("bf16_f128", T=128, d=512, F=64, E=8, k=2,
                                     capacity_factor=1.0, bias=SKEW_BIAS),
    # the K-part router (E = 8 or 16, T * E <= 64): 8 parts of 512 columns
    # (two runs per lane), a token bound above T, a score bias
    "bf16_parts_T5_bias": Workload("bf16_p5", T=5, d=4096, F=64, E=8, k=2,
                                   capacity_factor=1.0, bias=SKEW_BIAS),
    # 5 parts of 128 columns, T at the token bound
    "bf16_parts_T8_d640": Workload("bf16_p8", T=8, d=640, F=64, E=8, k=2),
    # the narrow MFMA router (E a multiple of 8 up to 64, beyond the K-part
    # router's batches): one, two and four 16-expert column fragments,
    # ragged last token groups, a score bias
    "bf16_narrow_E16": Workload("bf16_n16", T=333, d=384, F=64, E=16, k=4,
                                gating=SOFTMAX_THEN_TOPK, renormalize=False),
    "bf16_narrow_E24_bias": Workload("bf16_n24", T=190, d=640, F=64, E=24, k=3,
                                     capacity_factor=1.0, bias=(2.0,) * 3 + (0.0,) * 21),
    "bf16_narrow_E64": Workload("bf16_n64", T=257, d=1024, F=64, E=64, k=6,
                                gating=SOFTMAX_THEN_TOPK, renormalize=False),
    # d not a multiple of 256: 3 parts of 448 columns, a full chunk of K
    # steps and a 6-step tail per part
    "bf16_narrow_long_parts": Workload("bf16_nlong", T=17000, d=1344, F=64, E=8, k=2,
                                       capacity_factor=1.25),
}


@pytest.mark.parametrize("case", sorted(ROUTE_CASES))
def test_route_router_gemm(case):
    w = ROUTE_CASES[case]
    say(f"[route] {case}")
    run = Run(w)
    g, st = run.route()
    ref = run.oracle(tokens=[])
    Lg = g["logits"].numpy().astype(np.float64)
    scale = float(np.max(np.abs(ref["logits"])))
    err = float(np.max(np.abs(Lg - ref["logits"])))
    assert err <= (1e-5 if w.dtype == "bf16" else 1e-5) * max(1.0, scale) * math.sqrt(w.d / 64)
    ties, _, thr = near_tie_tokens(Lg, ref)
    ok = np.ones(w.T, dtype=bool)
    ok[ties] = False
    assert np.array_equal(g["idx"].numpy()[ok].astype(np.int64), ref["sel"][ok])
    if len(ties) == 0:
        assert np.array_equal(g["counts"].numpy().astype(np.int64), ref["dispatch"]["counts"])
        assert np.array_equal(g["slot"].numpy().astype(np.int64), ref["dispatch"]["slot"])
    say(f"  ok: logit err {err:.2e}, near ties {len(ties)} (thr {thr:.1e})")


# --------------------------------------------------------------------------
# full layer, every output element
# --------------------------------------------------------------------------
FORWARD_CASES = {
    "tiny_f32": PRESETS["tiny_f32"],
    "f32_shared_ragged": Workload("f32_shared", T=150, d=72, F=40, E=6, k=2, S=2,
                                  dtype="f32", capacity_factor=1.0),
    "bf16_multi_tile": Workload("bf16_multi", T=1000, d=256, F=512, E=8, k=2,
                                capacity_factor=1.25),
    "bf16_skew_drops": Workload("bf16_skew", T=1000, d=256, F=384, E=8, k=2,
                                capacity_factor=1.0, bias=SKEW_BIAS),
    "bf16_deepseek_like": Workload("bf16_ds", T=256, d=256, F=128, E=32, k=6, S=2,
                                   gating=SOFTMAX_THEN_TOPK, renormalize=False),
    "bf16_ragged_n": Workload("bf16_ragged", T=130, d=192, F=320, E=4, k=2,
                              capacity_factor=1.5),
    "bf16_dense_k_eq_E": Workload("bf16_dense", T=64, d=128, F=128, E=4, k=4),
    "bf16_T1": Workload("bf16_T1", T=1, d=256, F=512, E=8, k=2),
    # >= 384 rows per expert: the two-workgroups-per-CU kernel shape
    "bf16_long_rows": Workload("bf16_long", T=1600, d=128, F=320, E=4, k=1,
                               capacity_factor=1.25),
    # short-batch tiles (32 rows): several tiles per expert, drops, ragged N
    "bf16_short_tiles": Workload("bf16_short", T=64, d=128, F=192, E=2, k=1,
                                 capacity_factor=0.9),
    # token rows gathered into the K-blocked copy, hidden rows K-blocked, with
    # a shared expert (its hidden rows K-blocked too) and ragged last M-tiles
    "bf16_long_rows_shared": Workload("bf16_long_sh", T=1600, d=192, F=320, E=4, k=1,
                                      S=1, capacity_factor=1.25),
    # a few hundred rows per expert: 64-deep K steps, token rows read in place,
    # hidden rows K-blocked; shared experts
    "bf16_mid_rows_shared": Workload("bf16_mid_sh", T=512, d=128, F=192, E=4, k=2, S=2,
                                     capacity_factor=1.25),
    # a few rows for each of several experts: short tiles with narrow weight tiles
    "bf16_decode_narrow": Workload("bf16_dec_nar", T=16, d=256, F=384, E=8, k=2),
    # over 1.5k rows per expert: token rows read in place, hidden rows K-blocked
    "bf16_many_rows": Workload("bf16_many", T=4096, d=128, F=128, E=2, k=1,
                               capacity_factor=1.0),
    # overflow sent to spare experts, or processed in later rounds
    "bf16_skew_reroute": Workload("bf16_skew_rr", T=1000, d=256, F=384, E=8, k=2,
                                  capacity_factor=1.0, bias=SKEW_BIAS, overflow=1),
    "bf16_skew_sequential": Workload("bf16_skew_seq", T=1000, d=256, F=384, E=8, k=2,
                                     capacity_factor=1.0, bias=SKEW_BIAS, overflow=2),
    "bf16_deepseek_reroute": Workload("bf16_ds_rr", T=256, d=256, F=128, E=32, k=6, S=2,
                                      gating=SOFTMAX_THEN_TOPK, renormalize=False,
                                      capacity_factor=1.0, overflow=1),
    "bf16_short_reroute": Workload("bf16_short_rr", T=64, d=128, F=192, E=4, k=2,
                                   capacity_factor=0.75, overflow=1),
    # every token's 12 choices among the same 12 of 32 experts: up to 12
    # overflow rows per token, more than the 8 best experts a row keeps
    # from one scan, so later rows of a token wait a round
    "bf16_reroute_k12": Workload("bf16_rr_k12", T=96, d=128, F=64, E=32, k=12,
                                 capacity_factor=1.0, overflow=1,
                                 bias=(4.0,) * 12 + (0.0,) * 20),
    "f32_reroute_shared": Workload("f32_rr", T=150, d=72, F=40, E=6, k=2, S=1, dtype="f32",
                                   capacity_factor=0.8, overflow=1),
    # 256 experts, top-8: most experts get a handful of rows
    "bf16_E256_k8": Workload("bf16_e256", T=200, d=128, F=128, E=256, k=8,
                             capacity_factor=1.0),
    # one token with shared experts, softmax over all (a fine-grained decode step)
    "bf16_T1_shared_ds": Workload("bf16_t1s", T=1, d=256, F=192, E=64, k=6, S=2,
                                  gating=SOFTMAX_THEN_TOPK, renormalize=False),
    # a short fine-grained batch: 8 tokens, 6 of 64 experts each
    "bf16_T8_fine": Workload("bf16_t8f", T=8, d=256, F=128, E=64, k=6, S=1,
                             gating=SOFTMAX_THEN_TOPK, renormalize=False),
    # one slot per expert: almost everything dropped
    "bf16_one_slot": Workload("bf16_1slot", T=300, d=128, F=128, E=8, k=2,
                              capacity_factor=0.01),
    # capacity above T: nothing can overflow
    "bf16_capacity_above_T": Workload("bf16_bigcap", T=100, d=128, F=128, E=4, k=2,
                                      capacity_factor=50.0),
    # both choices of late tokens overflow: each goes to a different spare
    "bf16_pair_reroute": Workload("bf16_pair_rr", T=600, d=128, F=128, E=8, k=2,
                                  capacity_factor=1.25, bias=(3.0, 3.0, 0.0, 0.0, 0.0, 0.0,
                                                              0.0, 0.0), overflow=1),
    # skewed routing with a tiny capacity, overflow sent to spare experts
    "bf16_skew_reroute_tight": Workload("bf16_skrt", T=512, d=128, F=128, E=8, k=2,
                                        capacity_factor=0.3, bias=SKEW_BIAS, overflow=1),
}


@pytest.mark.parametrize("case", sorted(FORWARD_CASES))
def test_forward_small(case):
    w = FORWARD_CASES[case]
    say(f"[forward] {case}")
    run = Run(w)
    e = check_layer(run, case, live_row_rms=case in LIVE_ROW_RMS_CASES)
    if w.overflow != O.OVERFLOW_DROP:
        # the case exercises its policy
        assert e["dropped"] + e["rerouted"] > 0 or w.overflow == O.OVERFLOW_SEQUENTIAL


def test_forward_empty():
    say("[forward] T=0")
    w = Workload("empty", T=0, d=128, F=128, E=8, k=2, capacity_factor=1.25)
    cfg = config_for(w, stream=None)
    out = torch.empty((0, w.d), dtype=torch.bfloat16, device=DEV)
    x = torch.empty((0, w.d), dtype=torch.bfloat16, device=DEV)
    Wg = torch.zeros((w.d, w.E), dtype=torch.bfloat16, device=DEV)
    W = torch.zeros((w.E, w.d, w.F), dtype=torch.bfloat16, device=DEV)
    st = moe.moe_forward(x, Wg, W, W, W, cfg, out, stats=True)
    assert st["capacity"] == 0 and st["dropped"] == 0 and st["aux_loss"] == 0.0


def test_forward_deterministic():
    w = FORWARD_CASES["bf16_skew_drops"]
    say("[determinism] bf16 skew with drops")
    run = Run(w)
    a, _ = run.forward(stats=False)
    b, _ = run.forward(stats=False)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# --------------------------------------------------------------------------
# full workload sizes
# --------------------------------------------------------------------------
FULL = ["tiny_f32", "mixtral_prefill", "mixtral_decode_t1", "mixtral_decode_t8",
        "mixtral_decode_t64", "skew_cf1.0", "skew_cf1.5", "deepseek", "skew_cf1.0:reroute",
        "deepseek:reroute", "skew_cf1.0:sequential", "deepseek:routed_only"]
_POLICY = {"reroute": O.OVERFLOW_REROUTE, "sequential": O.OVERFLOW_SEQUENTIAL}
# layers whose every token is compared; the 16384-token skewed layers are
# compared on SKEW_TOKENS tokens that include every drop and reroute class
SKEW_TOKENS = 4096


def _class_sample(routing, T, n, seed=0):
    """n tokens of a large batch: up to a fair share from every class a
    token's assignments fall in (all kept, first choice dropped, second
    dropped, all dropped, some rerouted, first/last token), filled up at
    random."""
    rng = np.random.default_rng(seed)
    D = routing["dispatch"]
    k = routing["sel"].shape[1]
    dropped = (D["slot"] < 0).reshape(T, k)
    moved = ((D["expert"] != routing["sel"].reshape(-1)) & (D["expert"] >= 0)).reshape(T, k)
    classes = [np.nonzero(~dropped.any(1) & ~moved.any(1))[0],
               np.nonzero(moved.any(1))[0],
               np.nonzero(dropped.all(1))[0]]
    for j in range(k):
        only_j = dropped[:, j] & (dropped.sum(1) == 1)
        classes.append(np.nonzero(only_j)[0])
    pick = {0, T - 1}
    share = n // (len(classes) + 1)
    for c in classes:
        if len(c):
            pick.update(rng.choice(c, size=min(share, len(c)), replace=False).tolist())
            pick.update((int(c[0]), int(c[-1])))
    rest = np.setdiff1d(np.arange(T), np.fromiter(pick, dtype=np.int64))
    if len(pick) < n:
        pick.update(rng.choice(rest, size=min(n - len(pick), len(rest)), replace=False).tolist())
    return sorted(pick), [len(c) for c in classes]


@pytest.mark.parametrize("name", FULL)
def test_forward_full_size(name):
    base, _, policy = name.partition(":")
    w = PRESETS[base]
    if policy == "routed_only":
        # the shared experts carry most of RMS(ref) in this layer (the routed
        # gates sum to about 0.2), so the routed part is also checked alone
        w = w.with_(S=0)
    elif policy:
        w = w.with_(overflow=_POLICY[policy])
    say(f"[full] {name}")
    run = Run(w, gen_device=DEV if w.dtype == "bf16" else "cpu")
    # The router on its own: fp32 scores against fp64 ones, and the choices
    # of every token whose decision margin exceeds the score error.
    g_route, _ = run.route()
    Lg = g_route["logits"].numpy().astype(np.float64)
    indep = run.oracle(tokens=[])
    scale = float(np.max(np.abs(indep["logits"])))
    lerr = float(np.max(np.abs(Lg - indep["logits"])))
    assert lerr <= 1e-5 * max(1.0, scale) * math.sqrt(w.d / 64)
    ties, _, thr = near_tie_tokens(Lg, indep)
    ok = np.ones(w.T, dtype=bool)
    ok[ties] = False
    assert np.array_equal(g_route["idx"].numpy()[ok].astype(np.int64), indep["sel"][ok])
    say(f"  router: score err {lerr:.2e}, {len(ties)} tokens within {thr:.1e} of a tie")
    del indep
    # The layer, every token (or the class sample), on the GPU's scores; bf16
    # layers run on packed weights, as the bench times them, and must give
    # the row-major forward's bits.
    tokens = None
    if w.T > SKEW_TOKENS:
        routing = run.oracle(tokens=[], logits=Lg)
        tokens, sizes = _class_sample(routing, w.T, SKEW_TOKENS)
        say(f"  {len(tokens)} tokens from classes of sizes {sizes}")
        del routing
    check_layer(run, name, packed=w.dtype == "bf16", tokens=tokens,
                also_row_major=w.dtype == "bf16", per_gate_mass=policy == "routed_only")


# --------------------------------------------------------------------------
# down projections split in two K parts to fill the last round of resident
# workgroups, cut where the tiles that exist call for (on an MI355X's 512
# slots): fewer tiles than slots (476, cut at 2/3 of K) and one round plus a
# small remainder (544, cut at 2/3); d = 4352 also gives the router 4 parts
# of 1088 columns (several rounds of in-flight K steps).  Packed weights,
# every element, and the row-major forward's bits.
# --------------------------------------------------------------------------
KCUT_CASES = {
    "below_one_round": Workload("bf16_kcut0", T=1536, d=4352, F=256, E=8, k=2,
                                capacity_factor=1.25),
    "one_round_plus": Workload("bf16_kcut1", T=1664, d=4352, F=256, E=8, k=2,
                               capacity_factor=1.25),
}


@pytest.mark.parametrize("case", sorted(KCUT_CASES))
def test_forward_down_projection_cut(case):
    w = KCUT_CASES[case]
    say(f"[kcut] {case}")
    run = Run(w)
    check_layer(run, f"kcut/{case}", packed=True, also_row_major=True)


# --------------------------------------------------------------------------
# both FFN paths: grouped (no K split) and streaming (K split as far as
# possible), every output element
# --------------------------------------------------------------------------
PATH_CASES = ["bf16_T1", "bf16_multi_tile", "bf16_deepseek_like", "bf16_skew_drops",
              "bf16_ragged_n", "bf16_short_tiles", "bf16_long_rows"]


@pytest.mark.parametrize("path", [moe.PATH_GROUPED, moe.PATH_STREAM], ids=["grouped", "stream"])
@pytest.mark.parametrize("case", PATH_CASES)
def test_forward_paths(case, path):
    w = FORWARD_CASES[case]
    say(f"[forward path={path}] {case}")
    run = Run(w)
    check_layer(run, f"{case}/path{path}", path=path)


def test_load_balance_trend_of_gpu_batches():
    # [Routing guide] "Key insights" item 3: the load-balancing loss's trend.
    # Ten batches whose bias toward expert 0 shrinks: the GPU's aux loss per
    # batch, and its trend through moe_lb_trend, against the oracle's.
    w = Workload("trend", T=2000, d=64, F=64, E=8, k=2, capacity_factor=1.25)
    cfg = config_for(w, stream=None)
    ws = moe.Workspace(moe.moe_workspace_size(cfg))
    ws.bind(cfg)
    r = route_buffers(w.T, w.E, w.k)
    gpu, ref = [], []
    for i, b in enumerate(np.linspace(3.0, 0.0, 10)):
        L = random_logits(w.T, w.E, seed=40 + i)
        L[:, 0] += float(b)
        st = moe.moe_route_logits(L.to(DEV), cfg, r["idx"], r["w"], r["counts"], r["offsets"],
                                  r["perm"], r["slot"], stats=True)
        L64 = L.to(torch.float64).numpy()
        sel, _ = O.topk_select(L64, w.k)
        D = O.dispatch(sel, w.E, O.capacity(w.T, w.k, w.E, w.capacity_factor))
        aux = O.routing_stats(D["counts"], D["kept"], O.softmax_all(L64), w.T, w.k, w.E)["aux_loss"]
        assert abs(st["aux_loss"] - aux) <= 1e-5 * aux
        gpu.append(st["aux_loss"])
        ref.append(aux)
    slope, mean = moe.moe_lb_trend(gpu)
    want = O.load_balance_trend(ref)
    assert slope < 0
    assert abs(slope - want["slope"]) <= 1e-4 * abs(want["slope"])
    assert abs(mean - want["mean"]) <= 1e-5 * want["mean"]
    say(f"  aux {gpu[0]:.4f} -> {gpu[-1]:.4f}, trend {slope:.4e} per step (oracle {want['slope']:.4e})")

"""Benchmark of the sparse MoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one full layer forward (router, top-k gating, capacity dispatch,
expert SwiGLU FFNs, shared experts, gate-weighted combine) over one batch of
seeded synthetic input already resident in HBM.  The default workload is the
Mixtral-shaped 2048-token prefill layer (d 4096, d_ff 14336, 8 experts, top-2,
capacity factor 1.25).  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X published peaks
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0

# HBM-side bytes per launch of the dominant kernel, from two rocprofv3 --pmc
# runs (FETCH_SIZE, then WRITE_SIZE) scaled by what the same counters read for
# a 1 GiB device copy in the same run (FETCH_SIZE x 2.0, WRITE_SIZE x 1.0 on
# MI355X).  Keyed by workload and by a digest of the sources that define that
# kernel and its launch: once one of them changes, the figure no longer
# describes the kernel and the bench reports null.
MEASURED_TRAFFIC = {
    # workload: (source digest, fetch bytes, write bytes) per launch of the
    # routed SwiGLU GEMM on packed weights (the default layout); the counter
    # summaries are kept beside the profiles
    "mixtral_prefill": ("1ee5ca5811ba4faf", 3942.88e6, 122.20e6),
    "deepseek": ("1ee5ca5811ba4faf", 5342.00e6, 75.63e6),
    "mixtral_decode_t64": ("1ee5ca5811ba4faf", 1886.95e6, 3.67e6),
}
# The sources that define the routed SwiGLU GEMM and its launch: the kernel,
# the M-tile list built by the routing passes, the plan and the shared headers.
SOURCE_FILES = ("routing.hip", "ffn_grouped.hip", "ffn_dma.h", "moe_api.cpp", "common.h",
                "kernels.h")


def source_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    d = os.path.join(ROOT, "sparse_mixture_experts_capacity_amd", "csrc")
    for f in SOURCE_FILES:
        with open(os.path.join(d, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mixtral_prefill")
    ap.add_argument("--path", default="auto", choices=["auto", "grouped", "stream"])
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured once into a HIP graph and replayed "
                         "(no per-kernel events; reported beside the eager figures)")
    ap.add_argument("--backward", action="store_true",
                    help="also time the router backward (moe_router_backward) after the forward")
    ap.add_argument("--capacity-factor", type=float, default=None,
                    help="override the workload's capacity factor")
    ap.add_argument("--overflow", default="drop", choices=["drop", "reroute", "sequential"],
                    help="what happens to assignments beyond an expert's capacity")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=0)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--weights", default="packed", choices=["packed", "row_major"],
                    help="expert weight layout: packed once before timing (moe_pack_weights, "
                         "not timed) or the row-major tensors as generated")
    ap.add_argument("--cold-steps", type=int, default=10,
                    help="after the timed steps, this many more with L2 and the 256 MB "
                         "Infinity Cache flushed before each (reported separately)")
    ap.add_argument("--flush-mib", type=int, default=512)
    ap.add_argument("--decode-legs", default=None,
                    help="comma-separated token counts of extra decode steps timed on the same "
                         "weights (no capacity limit; default 1,64 for the Mixtral-shaped "
                         "prefill workload, none otherwise; 'none' for none)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one device copy of this many MiB before the steps "
                         "(a kernel of known traffic for scaling HBM counters)")
    return ap.parse_args()


def percentile(sorted_vals, q):
    """q-th percentile (0..100) of a sorted list, linear interpolation."""
    if not sorted_vals:
        return float("nan")
    pos = (len(sorted_vals) - 1) * q / 100.0
    lo = int(pos)
    hi = min(lo + 1, len(sorted_vals) - 1)
    return sorted_vals[lo] + (sorted_vals[hi] - sorted_vals[lo]) * (pos - lo)


def algorithmic_work(w, kept: int, hit_experts: int):
    """Flops and bytes the layer must do (no padding, no dropped rows, no
    unhit experts, no intermediates)."""
    es = 4 if w.dtype == "f32" else 2
    ffn_flops_per_row = 2 * 3 * w.d * w.F
    flops = (ffn_flops_per_row * kept + ffn_flops_per_row * w.S * w.T
             + 2 * w.T * w.d * w.E)
    weight_bytes = es * 3 * w.d * w.F * (hit_experts + w.S)
    io_bytes = es * (2 * w.T * w.d + w.d * w.E)
    gemm1_flops = 2 * w.d * 2 * w.F * kept
    gemm1_bytes = es * 2 * w.d * w.F * hit_experts
    # token rows read (each kept assignment once) and hidden rows written
    gemm1_io_bytes = es * kept * (w.d + w.F)
    return dict(flops=flops, bytes=weight_bytes + io_bytes, gemm1_flops=gemm1_flops,
                gemm1_bytes=gemm1_bytes, gemm1_io_bytes=gemm1_io_bytes)


def cpu_baseline(w, inp, n_tokens: int):
    """Time the fp64 oracle on the host: routing and dispatch of all T tokens,
    expert outputs for a seeded sample of n_tokens tokens."""
    import numpy as np
    import torch

    import oracle.oracle as O

    # threads the oracle's BLAS actually uses, the host's logical CPUs and
    # its CPU model
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    hx = inp.x.cpu()
    hWg = inp.W_gate.cpu()
    W1, W3, W2 = inp.W1.cpu(), inp.W3.cpu(), inp.W2.cpu()
    bias = None if inp.bias is None else inp.bias.cpu().double().numpy()

    def w64(t):
        return t.to(torch.float64).numpy()

    rng = np.random.default_rng(0)
    order = rng.permutation(w.T).tolist()   # the sample is a prefix of one seeded order
    shape = O.LayerShape(T=w.T, d=w.d, F=w.F, E=w.E, k=w.k, S=w.S, gating=w.gating,
                         renormalize=w.renormalize, capacity_factor=w.capacity_factor,
                         overflow=w.overflow)
    x64, wg64 = w64(hx), w64(hWg)
    experts = lambda e: (w64(W1[e]), w64(W3[e]), w64(W2[e]))  # noqa: E731
    # routing, dispatch and statistics alone (all T tokens, no expert outputs)
    t0 = time.perf_counter()
    O.forward(x64, shape, experts, W_gate=wg64, bias=bias, tokens=[])
    dt_route = time.perf_counter() - t0
    def timed(n):
        toks = sorted(order[:min(n, w.T)])
        t0 = time.perf_counter()
        O.forward(x64, shape, experts, W_gate=wg64, bias=bias, tokens=toks)
        return toks, time.perf_counter() - t0

    if n_tokens > 0:
        toks, dt = timed(n_tokens)
    else:
        # Size the sample for about 12 s of oracle work: two short runs give
        # the cost per token beyond the fixed cost of widening the weights.
        ta = timed(32)[1]
        tb = timed(64)[1]
        slope = (tb - ta) / 32
        n = w.T if slope <= 0 else int(64 + max(0.0, 12.0 - tb) / slope)
        toks, dt = timed(max(64, min(n, w.T)))
    return dict(value=len(toks) / dt, unit="tokens/s", cores=int(cores), kind="oracle",
                cpu_model=cpu_model, cpu_count=os.cpu_count(),
                sample=(f"{w.name}: routing, capacity dispatch and statistics of all {w.T} "
                        f"tokens plus expert and shared-expert outputs of {len(toks)} "
                        f"seeded sampled tokens, fp64 NumPy on the host; value = "
                        f"{len(toks)} tokens / {dt:.2f} s wall"),
                routing_seconds=dt_route, seconds=dt)


def decode_leg(moe, w, inp, weights, packed, T, stream, args, dom):
    """One decode batch of T tokens on workload w's weights (no capacity
    limit): ms per step (wall clock over K steps), the routed SwiGLU GEMM's
    time from HIP events in those steps, HBM fractions of the GEMM and of
    the layer, and a graph replay of the step."""
    import torch
    dev = "cuda"
    wd = w.with_(T=T, capacity_factor=0.0)
    cfg = moe.make_config(T=T, d_model=w.d, d_ff=w.F, n_experts=w.E, top_k=w.k,
                          n_shared=w.S, gating=w.gating, renormalize=w.renormalize,
                          capacity_factor=0.0, dtype=w.dtype, logit_bias=inp.bias,
                          stream=stream, overflow=w.overflow,
                          weight_layout=moe.WEIGHTS_PACKED if packed else moe.WEIGHTS_ROW_MAJOR)
    ws = moe.Workspace(moe.moe_workspace_size(cfg))
    ws.bind(cfg)
    x = inp.x[:T].contiguous()
    out = torch.empty((T, w.d), dtype=w.torch_dtype, device=dev)

    def step(stats=False):
        return moe.moe_forward(x, inp.W_gate, *weights, cfg, out, stats=stats)

    st = step(stats=True)
    for _ in range(args.warmup):
        step()
    stream.synchronize()
    moe.moe_timing_reset()
    moe.moe_timing_only(dom)
    moe.moe_timing_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    stream.synchronize()
    t1 = time.perf_counter()
    moe.moe_timing_enable(False)
    n_dom, t_dom = moe.moe_timing_read().get(dom, (0, 0.0))
    ms = (t1 - t0) * 1e3 / args.steps
    dom_ms = t_dom / n_dom if n_dom else float("nan")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step()
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    g0 = time.perf_counter()
    for _ in range(args.steps):
        g.replay()
    torch.cuda.synchronize()
    graph_ms = (time.perf_counter() - g0) * 1e3 / args.steps
    del g
    kept = int(sum(st["kept"]))
    hit = int(sum(1 for c in st["kept"] if c > 0))
    work = algorithmic_work(wd, kept, hit)
    g1_bytes = work["gemm1_bytes"] + work["gemm1_io_bytes"]
    return dict(
        workload=f"{w.name} weights, first {T} token rows, no capacity limit",
        T=T, ms_per_step=ms, tokens_per_s=T / (ms * 1e-3), graph_ms_per_step=graph_ms,
        experts_hit=hit, kept_assignments=kept,
        layer_bytes=work["bytes"],
        layer_frac_of_hbm=work["bytes"] / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        layer_frac_of_hbm_graph=work["bytes"] / (graph_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        dominant_kernel=dom, dominant_kernel_ms=dom_ms, dominant_kernel_bytes=g1_bytes,
        dominant_kernel_frac_of_hbm=g1_bytes / (dom_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        kernel_ms_source="HIP events around this kernel in each timed step")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path "
              f"(--gpus {args.gpus} requested)", file=sys.stderr)
        sys.exit(2)
    import torch

    import sparse_mixture_experts_capacity_amd as moe
    from workloads import PRESETS, make_inputs

    w = PRESETS[args.workload]
    overflow = {"drop": 0, "reroute": 1, "sequential": 2}[args.overflow]
    if overflow:
        w = w.with_(overflow=overflow)
    if args.capacity_factor is not None:
        w = w.with_(capacity_factor=args.capacity_factor)
    dev = "cuda"
    torch.cuda.init()
    inp = make_inputs(w, seed=args.seed, device=dev)
    path = {"auto": moe.PATH_AUTO, "grouped": moe.PATH_GROUPED, "stream": moe.PATH_STREAM}[args.path]
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        packed = args.weights == "packed" and w.dtype == "bf16"
        cfg = moe.make_config(T=w.T, d_model=w.d, d_ff=w.F, n_experts=w.E, top_k=w.k,
                              n_shared=w.S, gating=w.gating, renormalize=w.renormalize,
                              capacity_factor=w.capacity_factor, dtype=w.dtype,
                              ffn_path=path, logit_bias=inp.bias, stream=stream,
                              overflow=w.overflow,
                              weight_layout=moe.WEIGHTS_PACKED if packed else moe.WEIGHTS_ROW_MAJOR)
        ws = moe.Workspace(moe.moe_workspace_size(cfg))
        ws.bind(cfg)
        out = torch.empty((w.T, w.d), dtype=w.torch_dtype, device=dev)
        W1, W3, W2 = inp.W1, inp.W3, inp.W2
        if packed:
            # once, as a server would at load time; not part of any timing
            w13, w2b = moe.moe_packed_weight_bytes(cfg)
            W1 = torch.empty(w13 // 2, dtype=torch.bfloat16, device=dev)
            W3 = torch.empty(w13 // 2, dtype=torch.bfloat16, device=dev)
            W2 = torch.empty(w2b // 2, dtype=torch.bfloat16, device=dev)
            moe.moe_pack_weights(inp.W1, inp.W3, inp.W2, cfg, W1, W3, W2)
            stream.synchronize()

        def step(stats=False):
            return moe.moe_forward(inp.x, inp.W_gate, W1, W3, W2, cfg, out, stats=stats)

        if args.copy_calibration_mib:
            n = args.copy_calibration_mib * (1 << 20) // 4
            src = torch.randn(n, device=dev)
            dst = torch.empty_like(src)
            dst.copy_(src)
            stream.synchronize()
            del src, dst
        st = step(stats=True)   # routing statistics of this batch (not timed)
        for _ in range(args.warmup):
            step()
        stream.synchronize()
        # Timed region: only the dominant kernel (the routed SwiGLU GEMM) is
        # bracketed by the library's events, so the step carries two event
        # records and not two per kernel.
        dom = "ffn1_swiglu" if w.dtype == "bf16" else "ffn1_swiglu_f32"
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        moe.moe_timing_reset()
        moe.moe_timing_only(dom)
        moe.moe_timing_enable(True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            ev[i][0].record(stream)
            step()
            ev[i][1].record(stream)
        stream.synchronize()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        moe.moe_timing_enable(False)
        kern_timed = moe.moe_timing_read()
        step_ms = sorted(a.elapsed_time(b) for a, b in ev)
        # Breakdown: the same number of steps again with every kernel timed
        # (not part of the figure above).
        moe.moe_timing_reset()
        moe.moe_timing_only(None)
        moe.moe_timing_enable(True)
        for i in range(args.steps):
            step()
        stream.synchronize()
        moe.moe_timing_enable(False)
        kern = moe.moe_timing_read()

        # The same step captured into a graph and replayed: the launches of
        # one step go to the GPU as one submission.
        graph = None
        if args.graph:
            g = torch.cuda.CUDAGraph()
            stream.synchronize()
            with torch.cuda.graph(g, stream=stream):
                step()
            for _ in range(args.warmup):
                g.replay()
            torch.cuda.synchronize()
            g0 = time.perf_counter()
            for _ in range(args.steps):
                g.replay()
            torch.cuda.synchronize()
            graph = dict(ms_per_step=(time.perf_counter() - g0) * 1e3 / args.steps,
                         steps=args.steps)
            del g

        # Router backward (not part of the forward's timed region): after one
        # forward on this workspace, K timed backward calls with every output.
        bwd = None
        if args.backward:
            step()
            gen = torch.Generator(device=dev).manual_seed(1234)
            dout = torch.randn((w.T, w.d), generator=gen, device=dev).to(w.torch_dtype)
            dl = torch.empty((w.T, w.E), dtype=torch.float32, device=dev)
            dWg = torch.empty((w.d, w.E), dtype=torch.float32, device=dev)
            db = torch.empty((w.E,), dtype=torch.float32, device=dev)
            dx = torch.empty((w.T, w.d), dtype=torch.float32, device=dev)

            def bstep():
                moe.moe_router_backward(inp.x, inp.W_gate, dout, cfg, dl, dWg, db, dx,
                                        aux_coef=0.01, entropy_coef=0.001)

            for _ in range(args.warmup):
                bstep()
            stream.synchronize()
            moe.moe_timing_reset()
            moe.moe_timing_enable(True)
            b0 = time.perf_counter()
            for _ in range(args.steps):
                bstep()
            stream.synchronize()
            b1 = time.perf_counter()
            moe.moe_timing_enable(False)
            bk = moe.moe_timing_read()
            bwd = dict(ms_per_call=(b1 - b0) * 1e3 / args.steps,
                       kernels={n: dict(launches=c, avg_ms=t / max(c, 1)) for n, (c, t) in bk.items()})

        # Cold steps (not part of the timed region above): a buffer larger than
        # L2 and the Infinity Cache is read before each step, so no weight
        # bytes survive from the previous step.  It is read, not written, so
        # the caches hold clean lines and the step pays no write-back.
        cold = None
        if args.cold_steps > 0:
            flush = torch.ones(args.flush_mib * (1 << 20) // 4, dtype=torch.float32, device=dev)
            sink = torch.zeros((), dtype=torch.float32, device=dev)
            sink += flush.sum()
            stream.synchronize()
            cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.cold_steps)]
            moe.moe_timing_reset()
            moe.moe_timing_enable(True)
            for i in range(args.cold_steps):
                sink += flush.sum()
                cev[i][0].record(stream)
                step()
                cev[i][1].record(stream)
            stream.synchronize()
            moe.moe_timing_enable(False)
            ckern = moe.moe_timing_read()
            cold = dict(steps=args.cold_steps, flush_mib=args.flush_mib,
                        step_ms_median=percentile(sorted(a.elapsed_time(b) for a, b in cev), 50),
                        kernels={n: (t / c if c else 0.0) for n, (c, t) in ckern.items()})
            del flush, sink

        # Decode legs: the same expert weights (and the first T token rows)
        # at decode batch sizes with no capacity limit, each timed like the
        # main step (only the routed SwiGLU GEMM bracketed by events), plus a
        # graph replay of the step.  Not part of the headline figure.
        legs = {}
        leg_ts = args.decode_legs
        if leg_ts is None:
            leg_ts = "1,64" if w.name == "mixtral_prefill" else ""
        if leg_ts.strip().lower() == "none":
            leg_ts = ""
        for T in [int(v) for v in leg_ts.split(",") if v.strip()]:
            legs[f"t{T}"] = decode_leg(moe, w, inp, (W1, W3, W2), packed, T, stream, args, dom)

    ms = (t1 - t0) * 1e3 / args.steps
    kept = int(sum(st["kept"]))
    hit = int(sum(1 for c in st["kept"] if c > 0))
    work = algorithmic_work(w, kept, hit)
    per_kernel = {name: dict(launches=n, avg_ms=tot / max(n, 1) if n else 0.0)
                  for name, (n, tot) in kern.items()}
    # The routed SwiGLU GEMM (W1 and W3 of every hit expert) dominates every
    # workload.  Its bound is whichever floor is higher: the weight and row
    # bytes at peak HBM bandwidth, or its flops at peak MFMA rate (few rows per
    # expert, as in decode or with many fine-grained experts: HBM).
    n_dom, t_dom = kern_timed.get(dom, (0, 0.0))
    dom_ms = t_dom / n_dom if n_dom else float("nan")
    digest = source_digest()
    meas = (MEASURED_TRAFFIC.get(w.name)
            if w.overflow == 0 and args.capacity_factor is None and packed else None)
    traffic = None
    if meas is not None and meas[0] == digest:
        traffic = meas[1] + meas[2]
    peak_flops = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    g1_bytes = work["gemm1_bytes"] + work["gemm1_io_bytes"]
    hbm_bound = g1_bytes / (PEAK_HBM_GBS * 1e9) > work["gemm1_flops"] / (peak_flops * 1e12)
    if hbm_bound:
        achieved = g1_bytes / (dom_ms * 1e-3) / 1e9
        roof = dict(kernel=dom, bound="hbm", achieved=achieved, peak=PEAK_HBM_GBS,
                    unit="GB/s", frac=achieved / PEAK_HBM_GBS, traffic=traffic,
                    per_launch=(f"{g1_bytes} bytes (W1+W3 of {hit} hit experts, {kept} token "
                                f"rows read, {kept} hidden rows written)"))
    else:
        achieved = work["gemm1_flops"] / (dom_ms * 1e-3) / 1e12
        roof = dict(kernel=dom, bound="mfma", achieved=achieved, peak=peak_flops,
                    unit="TFLOP/s", frac=achieved / peak_flops, traffic=traffic,
                    per_launch=f"{work['gemm1_flops']} flops (2*d*2F per kept row, {kept} rows)")
    roof["kernel_ms"] = dom_ms
    roof["kernel_ms_source"] = ("HIP events around this kernel in each timed step "
                                "(the only kernel timed there)")
    roof["algorithmic_bytes"] = g1_bytes
    roof["traffic_unit"] = "bytes per launch (HBM side, counters)"
    roof["source_digest"] = digest
    if cold is not None:
        cold_dom = cold["kernels"].get(dom, float("nan"))
        cold_ach = (g1_bytes / (cold_dom * 1e-3) / 1e9 if hbm_bound
                    else work["gemm1_flops"] / (cold_dom * 1e-3) / 1e12)
        roof["cold"] = dict(kernel_ms=cold_dom, achieved=cold_ach, frac=cold_ach / roof["peak"],
                            note=f"L2 and Infinity Cache flushed ({cold['flush_mib']} MiB "
                                 f"read) before each of {cold['steps']} extra steps")
    # The pages' "dispatch time share" on one GPU: the time spent routing,
    # dispatching, gathering and combining rows, as a share of all the
    # layer's kernel time (the experts' GEMMs are the rest).
    route_names = ("router", "topk_gate", "route_small", "dispatch", "gather", "combine")
    kern_total = sum(v["avg_ms"] * v["launches"] for v in per_kernel.values()) / args.steps
    route_ms = sum(per_kernel[n]["avg_ms"] * per_kernel[n]["launches"]
                   for n in route_names if n in per_kernel) / args.steps
    layer_tflops = work["flops"] / (ms * 1e-3) / 1e12
    layer_gbs = work["bytes"] / (ms * 1e-3) / 1e9
    res = {
        "metric": "MoE-layer tokens/s",
        "value": w.T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded Gaussian inputs and weights of the workload's shapes)",
        "config": {"workload": w.name, "T": w.T, "d_model": w.d, "d_ff": w.F,
                   "n_experts": w.E, "top_k": w.k, "n_shared": w.S,
                   "capacity_factor": w.capacity_factor, "overflow": args.overflow,
                   "gating": "softmax_then_topk" if w.gating else "topk_then_softmax",
                   "weights": "packed" if packed else "row_major",
                   "parallelism": "single GPU"},
        "roofline": roof,
        "layer": {"active_tflops": layer_tflops,
                  "active_frac_of_bf16_peak": layer_tflops / PEAK_BF16_TFLOPS,
                  "algorithmic_gbs": layer_gbs,
                  "frac_of_hbm_peak": layer_gbs / PEAK_HBM_GBS,
                  "routing_ms": route_ms,
                  "routing_time_share": route_ms / kern_total if kern_total > 0 else None,
                  "kept_assignments": kept, "experts_hit": hit,
                  "capacity": st["capacity"], "dropped": st["dropped"],
                  "overflowed": st["overflowed"], "rerouted": st["rerouted"],
                  "rounds": st["rounds"],
                  "aux_loss": st["aux_loss"], "overflow_rate": st["overflow_rate"],
                  "entropy_load": st["entropy_load"], "entropy_token": st["entropy_token"],
                  "counts": [int(c) for c in st["counts"]]},
        "kernels": per_kernel,
        "kernels_source": ("a second pass of as many steps with every kernel bracketed "
                           "by HIP events; not part of ms_per_step"),
        "step_ms": {"median": percentile(step_ms, 50), "p10": percentile(step_ms, 10),
                    "p90": percentile(step_ms, 90), "source": "HIP events around each timed step"},
        "cold": cold,
    }
    if graph is not None:
        graph["tokens_per_s"] = w.T / (graph["ms_per_step"] * 1e-3)
        res["graph"] = graph
    if legs:
        res["decode"] = legs
    if bwd is not None:
        # The gate pass streams the kept expert rows and dout once: it is
        # bound by HBM.  Algorithmic bytes count each row in the layer's
        # dtype (the library keeps them in bf16, or as fp32 K parts when the
        # down projection is split).
        es = 2 if w.dtype == "bf16" else 4
        gbytes = kept * w.d * es + w.T * w.d * es + 2 * w.T * w.E * 4 + 3 * w.T * w.k * 4
        gms = bwd["kernels"].get("gate_backward", {}).get("avg_ms", float("nan"))
        gach = gbytes / (gms * 1e-3) / 1e9
        bwd["roofline"] = dict(kernel="gate_backward", bound="hbm", achieved=gach,
                               peak=PEAK_HBM_GBS, unit="GB/s", frac=gach / PEAK_HBM_GBS,
                               per_launch=(f"{gbytes} bytes ({kept} expert rows and the "
                                           f"dout rows in the layer dtype, scores and score "
                                           f"gradients)"))
        res["router_backward"] = bwd
    if not args.no_cpu_baseline:
        cb = cpu_baseline(w, inp, args.cpu_sample_tokens)
        res["cpu_baseline"] = {k: cb[k] for k in ("value", "unit", "cores", "kind", "sample",
                                                   "cpu_model", "cpu_count")}
        res["cpu_baseline"]["routing_dispatch_stats_s"] = cb["routing_seconds"]
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

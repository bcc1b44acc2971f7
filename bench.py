#!/usr/bin/env python3
"""Benchmark of the LatentMoE layer forward on one MI355X.

One step = one full layer forward (all stages: W_down + router GEMMs, top-k
and gates, dispatch indices, grouped FC1 + activation, grouped FC2, combine,
W_up, and the shared experts when the workload has them, by default on a
side stream) over one batch of synthetic tokens already resident in HBM.

The default run is the suite of the five layer configurations.  The JSON
line's headline is the largest one, the 512-expert top-22 prefill layer
(T 16384, d 4096, l 1024, m 2048: MFMA-bound); the line's "configs" object
holds the same measurement for the other four (the tiny fp32 layer, the
standard-MoE and LatentMoE decode layers, the fp8 896-expert layer).  Each
carries tokens/s, ms per step, latency percentiles, the roofline of its
dominant kernel (from HIP events the library records on the launch stream
around each stage) and the fp64 CPU oracle's throughput on a bounded token
sample.  --workload W runs one workload alone.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}
HEADLINE = "latent_prefill_zipf"
SUITE = ("latent_prefill_zipf", "tiny", "std_decode", "latent_decode", "latent_fp8_sparse",
         "latent_mxfp4_decode")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def expert_weight_bytes(spec, counts, stage):
    """Expert-weight bytes one expert-FFN launch must read: both matrices
    of every expert that received tokens for the fused kernel (stage
    "ffn"), one matrix for FC1 / FC2 (SwiGLU FC1: up and gate rows), fp8
    row scales and MXFP4 block scales included.  Token rows, H and Y are
    intermediates and are not counted."""
    touched = int((counts > 0).sum())
    eb = spec.expert_bytes
    l, m = spec.l, spec.m
    m1 = 2 * m if spec.activation == "swiglu" else m
    w1 = touched * l * m1 * eb
    w2 = touched * l * m * eb
    if spec.expert_dtype == "fp8_e4m3_rowscale":
        w1 += touched * m1 * 4
        w2 += touched * l * 4
    return float({"ffn": w1 + w2, "fc1": w1, "fc2": w2}[stage])


def expert_kernel_work(spec, T, counts, stage):
    """Algorithmic bytes (expert weights, expert_weight_bytes) and FLOPs
    (2 * T*K * l * m per GEMM, SwiGLU FC1 twice that) of one FC1 or FC2
    launch, or of the fused FC1 + FC2 kernel (stage "ffn")."""
    l, m, K = spec.l, spec.m, spec.top_k
    m1 = 2 * m if spec.activation == "swiglu" else m
    flops = {"ffn": 2.0 * T * K * l * (m1 + m), "fc1": 2.0 * T * K * l * m1,
             "fc2": 2.0 * T * K * l * m}[stage]
    return expert_weight_bytes(spec, counts, stage), flops


def layer_work(spec, T, counts):
    """Algorithmic bytes and FLOPs of one whole layer call: weights of the
    experts that received tokens, projections and router read once, x read
    once, out written once (permuted copies, H, Y and logits are
    intermediates a fused implementation keeps on chip, so they are not
    counted); FLOPs 2*T*d*l per projection, 2*T*r_in*N for the router,
    4*T*K*l*m for the routed experts and 4*T*d*S*m_s for the shared ones
    (whose weights, 2*d*S*m_s elements, are read once); SwiGLU experts have
    a third matrix of the FC1 shape (6*T*K*l*m, 3*d*S*m_s)."""
    d, l, m, N, K = spec.d, spec.l, spec.m, spec.n_experts, spec.top_k
    a, eb = spec.act_bytes, spec.expert_bytes
    r_in = l if spec.router_on_latent else d
    touched = int((counts > 0).sum())
    nmat = 3 if spec.activation == "swiglu" else 2   # m x l matrices per expert
    per_expert = nmat * l * m * eb
    if spec.expert_dtype == "fp8_e4m3_rowscale":
        per_expert += 4.0 * ((nmat - 1) * m + l)
    nbytes = touched * per_expert + N * r_in * a + 2.0 * T * d * a
    if spec.has_router_bias:
        nbytes += 4.0 * N
    flops = 2.0 * T * r_in * N + 2.0 * nmat * T * K * l * m
    if spec.has_projections:
        nbytes += 2.0 * l * d * a
        flops += 4.0 * T * d * l
    hs = spec.n_shared * spec.m_shared
    nbytes += nmat * d * hs * a
    flops += 2.0 * nmat * T * d * hs
    return nbytes, flops


def cpu_baseline(spec, w_np, x_np, budget_s=10.0, threads=None):
    """The fp64 oracle on the first n tokens of the batch, n sized so that the
    run takes about budget_s seconds on `threads` host threads (default: the
    OpenMP default, all host cores)."""
    import oracle
    T = x_np.shape[0]
    default = oracle.max_threads()
    if threads:
        oracle.set_threads(threads)
    used = oracle.max_threads()
    try:
        n = min(T, 2 * used)                          # probe: two tokens per thread
        t0 = time.perf_counter()
        oracle.forward(spec, w_np, x_np, tokens=list(range(n)))
        dt = time.perf_counter() - t0
        per_tok = max(dt / n, 1e-7)
        n2 = int(min(T, max(n, budget_s / per_tok)))
        reps, dt2 = 0, 0.0
        # a batch much shorter than the budget (the tiny layer) is repeated
        while reps == 0 or (n2 == T and dt2 < 0.5 * budget_s):
            t0 = time.perf_counter()
            oracle.forward(spec, w_np, x_np, tokens=list(range(n2)))
            dt2 += time.perf_counter() - t0
            reps += 1
    finally:
        oracle.set_threads(default)
    what = ("the %d tokens of the batch, %d times" % (T, reps) if reps > 1 else
            "first %d of the %d tokens of the same batch" % (n2, T))
    return {"value": reps * n2 / dt2, "unit": "tokens/s", "cores": used, "kind": "oracle",
            "sample": "%s, full layer in fp64 (%.1f s)" % (what, dt2)}


def measure(name, args, tokens=0, cpu=True, cpu_budget=10.0):
    """One workload: inputs generated and moved to HBM, warmup, K timed
    steps, per-step latencies, per-stage event times, the roofline of the
    dominant kernel and of the whole step, and the oracle's CPU rate."""
    import numpy as np
    import torch
    import mixture_experts_layer_32_amd as pkg
    import synth

    wl = synth.workload(name)
    spec, T = wl.spec, (tokens or wl.T)
    dev = torch.device("cuda:0")
    log("bench: workload %s T=%d: generating inputs" % (wl.name, T))
    t0 = time.perf_counter()
    w_np = synth.make_weights(spec, seed=0)
    x_np = synth.make_tokens(spec, T, seed=0)
    d_all = pkg.to_device(pkg.pack_gated(dict(w_np, x=x_np)), dev)
    torch.cuda.synchronize()
    log("bench: inputs on device in %.1f s" % (time.perf_counter() - t0))

    layer = pkg.LatentMoELayer(spec, expert_kernel=args.expert_kernel)
    # the grouped expert kernels (bf16, fp8) read their weights from the
    # banded copy, made once here like any weight preparation before serving
    # (not timed)
    packed = layer.expert_regime(T) in ("grouped", "fp8w") and layer.packed_weights_size() > 0
    if packed:
        d_all["experts_packed"] = layer.pack_expert_weights(d_all)
        torch.cuda.synchronize()
    cw = layer.weights_struct(d_all)
    x = d_all["x"]
    act = torch.float32 if spec.act_dtype == "f32" else torch.bfloat16
    out = torch.empty((T, spec.d), dtype=act, device=dev)
    ws = torch.empty((layer.workspace_size(T),), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    overlap = pkg.Overlap(device=dev) if spec.n_shared and args.overlap == "on" else None

    def step(timer=None, debug=None):
        layer.forward(x, None, out=out, workspace=ws, cweights=cw, stream=stream, timer=timer,
                      debug=debug, overlap=overlap)

    dbg = {"expert_counts": torch.empty((spec.n_experts,), dtype=torch.int32, device=dev)}
    step(debug=dbg)
    torch.cuda.synchronize()
    counts = dbg["expert_counts"].cpu().numpy()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("bench: warmup done (%d steps)" % args.warmup)

    # timed region: K plain steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    log("bench: %.3f ms/step" % ms)

    # per-step latency distribution: one event pair around every step
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for a, b in evs:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    lat = np.sort(np.array([a.elapsed_time(b) for a, b in evs]))
    pct = {"p50": float(np.percentile(lat, 50)), "p95": float(np.percentile(lat, 95)),
           "p99": float(np.percentile(lat, 99)), "mean": float(lat.mean())}
    log("bench: latency ms " + " ".join("%s=%.4f" % kv for kv in pct.items()))

    # per-stage durations from HIP events recorded by the library on the launch stream
    timer = pkg.StageTimer()
    n_done, stage_ms = 0, {k: 0.0 for k in pkg.STAGE_NAMES}
    while n_done < args.steps:
        n = min(200, args.steps - n_done)
        for _ in range(n):
            step(timer=timer)
        got, calls = timer.read()
        for k in stage_ms:
            stage_ms[k] += got[k]
        n_done += calls
    stage_avg = {k: v / n_done for k, v in stage_ms.items()}
    timer.close()
    log("bench: stages (ms) " + " ".join("%s=%.4f" % kv for kv in stage_avg.items()))

    regime = layer.expert_regime(T)
    if regime == "fused":  # FC1 and FC2 in one kernel, launched in the FC1 stage
        dom = "ffn"          # (the FC2 stage then holds no kernel, only its events)
        t_dom_ms = stage_avg["fc1"]
    else:
        dom = "fc1" if stage_avg["fc1"] >= stage_avg["fc2"] else "fc2"
        t_dom_ms = stage_avg[dom]
    nbytes, nflops = expert_kernel_work(spec, T, counts, dom)
    t_dom = t_dom_ms * 1e-3
    mfma_peak = MFMA_PEAK_TFLOPS["f32" if spec.act_dtype == "f32" else "bf16"]
    if wl.regime == "prefill":
        # the expert contraction runs on bf16 MFMA: FLOPs of the layer's
        # definition (no tile padding) over the launch's duration
        roof = {"bound": "mfma", "achieved": round(nflops / t_dom / 1e12, 2),
                "peak": mfma_peak, "unit": "TFLOP/s"}
    else:
        # expert weights streamed from HBM (the decode layers, the fp8 layer;
        # the tiny fp32 layer is launch-latency bound and is reported the same way)
        roof = {"bound": "hbm", "achieved": round(nbytes / t_dom / 1e9, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    # measured HBM bytes per launch of this kernel (rocprofv3 FETCH_SIZE and
    # WRITE_SIZE, copy-calibrated), only while the kernel sources are the
    # ones the counters were taken on
    from mixture_experts_layer_32_amd import profiling
    hbm = profiling.read_hbm(wl.name, dom, regime) if T == wl.T else None
    roof["traffic"] = round(hbm) if hbm is not None else None
    roof["kernel"] = ("expert FFN, FC1 + FC2 (fused kernel)" if dom == "ffn" else
                      "expert GEMM %s (%s kernel)" % (dom.upper(), regime))
    roof["algorithmic_bytes_per_launch"] = nbytes
    roof["algorithmic_flops_per_launch"] = nflops
    roof["launch_ms"] = round(t_dom_ms, 5)
    if wl.regime == "tiny":
        roof["note"] = "parity configuration; launch-latency bound"

    # the whole step against both ceilings
    lb, lf = layer_work(spec, T, counts)
    layer_roof = {"algorithmic_bytes": lb, "algorithmic_flops": lf,
                  "hbm_frac": round(lb / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
                  "mfma_frac": round(lf / (ms * 1e-3) / (mfma_peak * 1e12), 4),
                  "mfma_peak_tflops": mfma_peak}

    res = {
        "metric": "MoE-layer tokens/s @1 GPU",
        "value": round(T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16"}[spec.act_dtype] + {
            "fp8_e4m3_rowscale": "+fp8w", "mxfp4_e2m1": "+mxfp4w"}.get(spec.expert_dtype, ""),
        "data": "synthetic (seeded normals, N(0,1/fan_in) weights)",
        "config": {"workload": wl.name, "T": T, "d": spec.d, "l": spec.l, "m": spec.m,
                   "n_experts": spec.n_experts, "top_k": spec.top_k, "gating": spec.gating,
                   "expert_dtype": spec.expert_dtype, "parallelism": "single GPU",
                   "n_shared": spec.n_shared, "m_shared": spec.m_shared,
                   "activation": spec.activation,
                   "shared_on_side_stream": overlap is not None,
                   "expert_kernel": regime,
                   "expert_weights": "banded copy" if packed else "row-major"},
        "stage_ms": {k: round(v, 5) for k, v in stage_avg.items()},
        "latency_ms": {k: round(v, 5) for k, v in pct.items()},
        "roofline": roof,
        "layer_roofline": layer_roof,
        "experts": {"touched": int((counts > 0).sum()),
                    "max_rows": int(counts.max()), "median_rows": float(np.median(counts))},
    }
    if spec.n_shared:
        # the shared experts' two dense GEMMs (their stage's events, on the
        # stream they ran on; beside the routed path they share the GPU)
        hs = spec.n_shared * spec.m_shared
        nmat = 3 if spec.activation == "swiglu" else 2
        sf = 2.0 * nmat * T * spec.d * hs
        t_sh = stage_avg["shared"] * 1e-3
        res["shared_stage"] = {"ms": round(stage_avg["shared"], 5), "algorithmic_flops": sf,
                               "tflops": round(sf / t_sh / 1e12, 2) if t_sh > 0 else None,
                               "mfma_frac": round(sf / t_sh / (mfma_peak * 1e12), 4)
                               if t_sh > 0 else None}
    del d_all, x, out, ws, cw, layer, overlap
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if cpu:
        log("bench: timing the fp64 CPU oracle")
        res["cpu_baseline"] = cpu_baseline(spec, w_np, x_np, cpu_budget)
        if wl.regime == "tiny":
            res["cpu_baseline_1core"] = cpu_baseline(spec, w_np, x_np, cpu_budget / 2, threads=1)
    return res


CONFIG_KEYS = ("value", "unit", "ms_per_step", "dtype", "config", "stage_ms", "latency_ms",
               "roofline", "layer_roofline", "experts", "cpu_baseline", "cpu_baseline_1core")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="suite",
                    help="'suite' (default: the five layer configurations, headline %s) or one "
                         "workload name" % HEADLINE)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of oracle work per configuration")
    ap.add_argument("--overlap", choices=("on", "off"), default="on",
                    help="shared experts on a side stream (on) or first on the launch stream")
    ap.add_argument("--tokens", type=int, default=0,
                    help="tokens per call (default: the workload's batch; single workloads only)")
    ap.add_argument("--expert-kernel", choices=("auto", "tiled", "stream", "fused"),
                    default="auto", help="force one expert-FFN kernel (default: the library's choice)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (known HBM traffic: "
                         "1 GiB read + 1 GiB written per launch) to scale rocprofv3 "
                         "FETCH_SIZE / WRITE_SIZE readings")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the layer is benchmarked on a single MI355X "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        a = torch.empty((1 << 30,), dtype=torch.uint8, device="cuda:0").fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read_per_launch": 1 << 30,
                          "bytes_written_per_launch": 1 << 30, "launches": 5}))
        return

    cpu = not args.no_cpu_baseline
    if args.workload != "suite":
        print(json.dumps(measure(args.workload, args, args.tokens, cpu, args.cpu_budget)),
              flush=True)
        return
    res = measure(HEADLINE, args, 0, cpu, args.cpu_budget)
    res["configs"] = {HEADLINE: {k: res[k] for k in CONFIG_KEYS if k in res}}
    for name in SUITE:
        if name == HEADLINE:
            continue
        r = measure(name, args, 0, cpu, args.cpu_budget)
        res["configs"][name] = {k: r[k] for k in CONFIG_KEYS if k in r}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Throughput of the MI355X MoE layer (gpt-oss MoE MLP) on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

With no --workload, every leg of the metric runs in turn and one JSON line is
printed: the headline is the 36-layer 120b stack (T 2048, E 128 -- the
largest configuration, HBM-bound), and "legs" holds the same record for the
20b decode batch (T 32, HBM-bound), the 20b prefill batch (T 4096,
MFMA-bound) and the 120b prefill batch with Zipf-skewed expert loads
(T 8192, E 128), plus the attention steps beside the layer (grouped-query
attention with sinks over a 128-position band or dense, at prefill and
decode sizes; --no-attention leaves them out).  --workload NAME runs that one
workload as the headline.

A step is one call of the whole layer -- router + top-k + softmax, expert
row lists, gate/up GEMM with the clamped-SwiGLU epilogue, down GEMM, weighted
combine -- on one batch of synthetic inputs already resident in HBM (for the
36-layer stack, one pass through all layers with the RMSNorm and residual
add between them).  Single-layer steps rotate over several independently
seeded weight sets so that HBM, not the 256 MB Infinity Cache, serves the
weights.  Every leg times exactly K steps after W warm-up steps, on the
expert weights in the library's packed layout (moe_pack_weights, applied
once per weight set before timing: the same MXFP4 bytes, two weight rows per
128-byte line); the same leg on the row-major stored layout is timed beside
it and reported under config.rowmajor.

Per-kernel durations come from HIP events the library records around its
launches on the launch stream (moe_timing_enable); the dominant kernel's
algorithmic bytes (HBM-bound legs) or FLOPs (MFMA-bound legs) divided by its
mean duration give the roofline fraction.  The CPU baseline times the fp64
oracle on a bounded sample of the same workload on this host.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + % roofline (HBM GB/s decode, MFMA TFLOPS prefill)"
HBM_PEAK = 8.0e12          # MI355X HBM3E, bytes/s
MFMA_FP6_FP4_PEAK = 10.1e15  # MI355X dense FP6/FP4 MFMA, FLOP/s
KEYS = ["x", "router_w", "router_b", "w13_codes", "w13_scales", "b13", "w2_codes", "w2_scales", "b2"]
LAYER_KEYS = KEYS[1:]
# legs of the default run: (workload, roofline bound); the last is the headline
LEGS = [("20b_decode", "hbm"), ("20b_prefill", "mfma"), ("120b_prefill_zipf", "mfma"), ("120b_stack36", "hbm")]
# the attention steps beside the layer, reported under "legs" (not the headline)
ATTN_LEGS = ["attn_prefill_band", "attn_prefill_dense", "attn_decode_dense", "attn_decode_band"]
BF16_MFMA_PEAK = 2.5e15    # MI355X dense bf16 MFMA, FLOP/s
TIME_EVERY = 10            # every TIME_EVERY-th timed step brackets the dominant kernel with events
SAMPLE_EXTRA = 200         # single-layer legs: more steps after the K timed ones, sampled the same way


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def mxfp4_bytes(rows: int, cols: int) -> int:
    return rows * cols // 2 + rows * cols // 32


def gen_layer(wl, seed, torch, keep_host=False):
    import numpy as np
    from moe_inputs import synth
    from moe_inputs.workloads import ZIPF_BETA
    x = synth.gen_x(seed, wl.T, wl.d)
    wr, br = synth.gen_router(seed, wl.E, wl.d)
    if wl.routing == "zipf":
        br = synth.zipf_router_bias(seed, wl.E, ZIPF_BETA)
    inp = dict(x=x, router_w=wr, router_b=br, **synth.gen_experts(seed, wl.E, wl.d, wl.I))
    out = {}
    for k in KEYS:
        a = np.ascontiguousarray(inp[k])
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if a.dtype == np.uint16 else torch.from_numpy(a)
        out[k] = t.to("cuda:0")
    return out, (inp if keep_host else None)


def read_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, or None when
    the summary is missing or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    from sparse_moe_transformer_softmax_amd.profsum import src_sha
    if kv.get("src_sha") != src_sha():
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def host_cpu():
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:  # pragma: no cover
        pass
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return model, n


def _oracle_rate(wl, inp, n, budget_s, act):
    """Tokens/s of the oracle on the first n tokens, repeated until about
    budget_s is spent; returns (rate, runs, seconds)."""
    from oracle import moe_oracle as O
    reps, total = 0, 0.0
    while reps == 0 or total < budget_s:
        t0 = time.perf_counter()
        O.moe_layer(inp["x"][:n], inp["router_w"], inp["router_b"], inp, wl.k, wl.clamp, act=act)
        total += time.perf_counter() - t0
        reps += 1
    return reps * n / total, reps, total


def cpu_baseline(wl, inp, budget_s: float, act: str = "exact"):
    """The fp64 oracle on a bounded sample of the workload's tokens, on this
    host: the sample doubles until one run takes a quarter of the budget,
    then repeats until about half of it is spent."""
    from oracle import moe_oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        blas = 1
    model, ncpu = host_cpu()
    n = 1
    while True:
        t0 = time.perf_counter()
        O.moe_layer(inp["x"][:n], inp["router_w"], inp["router_b"], inp, wl.k, wl.clamp, act=act)
        spent = time.perf_counter() - t0
        if spent > budget_s / 4 or n >= wl.T:
            break
        n = min(wl.T, 2 * n)
    rate, reps, total = _oracle_rate(wl, inp, n, budget_s / 2, act)
    note = f"; stack rate = one layer's rate / {wl.layers}" if wl.layers > 1 else ""
    return {"value": rate / wl.layers, "unit": "tokens/s", "cores": int(blas), "kind": "oracle",
            "cpu_model": model, "nproc": ncpu,
            "sample": f"first {n} tokens of weight set 0 through one layer, {reps} runs, fp64 numpy oracle "
                      f"({blas} BLAS threads), {total:.1f} s{note}"}


def one_thread_rates(budget_s: float):
    """The oracle on one thread for the tiny layer and the 20b decode batch."""
    from threadpoolctl import threadpool_limits
    from moe_inputs.workloads import WORKLOADS
    from oracle.workload_inputs import make_inputs
    out = {}
    with threadpool_limits(limits=1):
        for name, n in (("tiny", 16), ("20b_decode", 4)):
            wl = WORKLOADS[name]
            inp = make_inputs(wl, condition=False)
            rate, reps, total = _oracle_rate(wl, inp, n, budget_s, "exact")
            out[name] = {"value": rate, "unit": "tokens/s", "cores": 1,
                         "sample": f"first {n} tokens, {reps} runs, {total:.1f} s"}
    return out


def run_leg(wl, bound, args, torch, moe, want_cpu):
    """Times one workload; returns its record (metric fields, config,
    roofline, cpu_baseline)."""
    import numpy as np

    expert_bytes = mxfp4_bytes(2 * wl.I, wl.d) + mxfp4_bytes(wl.d, wl.I) + 4 * (2 * wl.I + wl.d)
    layer_weight_bytes = wl.E * expert_bytes
    nlay = wl.layers
    if args.sets:
        nsets = args.sets
    elif nlay > 1:
        nsets = 1
    else:
        nsets = max(1, min(4, int(np.ceil(1.1e9 / layer_weight_bytes))))
    log(f"workload {wl.name}: T={wl.T} d={wl.d} I={wl.I} E={wl.E} k={wl.k} layers={nlay} sets={nsets}")

    t0 = time.perf_counter()
    sets, host0 = [], None
    for s in range(nsets if nlay == 1 else nlay):
        g, h = gen_layer(wl, wl.seed + 1000 * s if nlay == 1 else wl.seed + s, torch, keep_host=(s == 0 and want_cpu))
        sets.append(g)
        if h is not None:
            host0 = h
    torch.cuda.synchronize()
    log(f"inputs generated and uploaded in {time.perf_counter() - t0:.1f} s")

    # routing of every set, for the algorithmic byte and FLOP counts
    n_sel = []
    for g in sets:
        _, _, counts = moe.moe_route(g["x"], g["router_w"], g["router_b"], k=wl.k)
        n_sel.append(int((counts > 0).sum().item()))
    P = wl.T * wl.k
    x_bytes = wl.T * wl.d * 2

    # Every leg runs on both weight layouts: the packed layout
    # (moe_pack_weights, once per weight set before timing) is the primary
    # record; the row-major layout (the stored format, moe_layer_forward)
    # is timed the same way beside it.
    t0 = time.perf_counter()
    psets = []
    for g in sets:
        pg = dict(g)
        pg["w13_codes"], pg["w13_scales"] = moe.moe_pack_weights(g["w13_codes"], g["w13_scales"])
        pg["w2_codes"], pg["w2_scales"] = moe.moe_pack_weights(g["w2_codes"], g["w2_scales"])
        psets.append(pg)
    torch.cuda.synchronize()
    log(f"weights packed in {time.perf_counter() - t0:.2f} s")
    act_flag = {"exact": 0, "mxfp6": moe.MOE_LAYER_MXFP6, "mx6x2": moe.MOE_LAYER_MX6X2}[args.act]

    def make_step(S, packed):
        flags = (moe.MOE_LAYER_PACKED if packed else 0) | act_flag
        if nlay == 1:
            outs = [torch.empty((wl.T, wl.d), dtype=torch.bfloat16, device="cuda:0") for _ in range(nsets)]

            def step(i):
                g = S[i % nsets]
                if flags:
                    return moe.moe_layer_forward_ex(*[g[k] for k in KEYS], k=wl.k, clamp=wl.clamp, flags=flags,
                                                    out=outs[i % nsets])
                return moe.moe_layer_forward(*[g[k] for k in KEYS], k=wl.k, clamp=wl.clamp, out=outs[i % nsets])
        else:
            x0 = S[0]["x"]
            out = torch.empty_like(x0)
            layers = [{k: g[k] for k in LAYER_KEYS} for g in S]

            def step(i):
                return moe.moe_stack_forward(x0, layers, k=wl.k, clamp=wl.clamp, eps=1e-5, out=out, flags=flags)
        return step

    def measure(step, breakdown):
        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
        kt = None
        if breakdown:
            # per-kernel breakdown (diagnostic, untimed): every kernel bracketed by events
            moe.moe_timing_read(reset=True)
            moe.moe_timing_enable(True)
            for i in range(min(args.steps, 20 if nlay == 1 else 2)):
                step(i)
            torch.cuda.synchronize()
            moe.moe_timing_enable(False)
            kt = moe.moe_timing_read(reset=True)
        # timed region: K steps; in every TIME_EVERY-th step the library
        # brackets the dominant kernel's launches (gate/up GEMM) with HIP
        # event pairs on the launch stream.  An event pair costs about 11 us
        # of stream time around a decode step, so bracketing every step would
        # inflate the step time it is measured in; the sampled launches run
        # inside the same stream of steps.  A single-layer leg then runs
        # SAMPLE_EXTRA more steps back to back in the same stream, sampled the
        # same way, so that the kernel's mean rests on more than K / 10
        # launches; the step time is that of the K steps alone.
        moe.moe_timing_read(reset=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        for i in range(args.steps):
            timed = i % TIME_EVERY == 0
            if timed:
                moe.moe_timing_enable(["gateup_gemm"])
            step(i)
            if timed:
                moe.moe_timing_enable(False)
        ev1.record()
        extra = SAMPLE_EXTRA if nlay == 1 else 0
        for i in range(args.steps, args.steps + extra):
            timed = i % TIME_EVERY == 0
            if timed:
                moe.moe_timing_enable(["gateup_gemm"])
            step(i)
            if timed:
                moe.moe_timing_enable(False)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        kt_live = moe.moe_timing_read(reset=True)
        ms_step = ev0.elapsed_time(ev1) / args.steps
        gu_ms, gu_n = kt_live["gateup_gemm"]
        return ms_step, wall / (args.steps + extra), gu_ms / max(gu_n, 1) * 1e3, gu_n, kt

    ms_rm, wall_rm, gu_us_rm, _, kt_rm = measure(make_step(sets, False), breakdown=True)
    log(f"row-major weights: {ms_rm * 1e3:.1f} us/step (host wall {wall_rm * 1e6:.1f} us/step), "
        f"gate/up live {gu_us_rm:.1f} us")
    for kname, (ms, n) in kt_rm.items():
        if n:
            log(f"  {kname:12s} {ms / n * 1e3:9.1f} us/launch  x{n}  (separate pass, all kernels timed)")
    ms_step, wall, gu_us, gu_n, kt = measure(make_step(psets, True), breakdown=True)
    tok_s = wl.T / (ms_step * 1e-3)
    log(f"packed weights: timed {args.steps} steps: {ms_step * 1e3:.1f} us/step "
        f"(host wall {wall * 1e6:.1f} us/step)")
    for kname, (ms, n) in kt.items():
        if n:
            log(f"  {kname:12s} {ms / n * 1e3:9.1f} us/launch  x{n}  (separate pass, all kernels timed)")
    log(f"  gateup_gemm live in the timed region: {gu_us:.1f} us/launch ({gu_n} sampled launches)")

    # algorithmic work
    if nlay == 1:
        nsel_mean = float(np.mean([n_sel[i % nsets] for i in range(args.steps)]))
        # the weight sets of the sampled gate/up launches (every TIME_EVERY-th
        # step of the K timed and SAMPLE_EXTRA further steps)
        nsel_gu = float(np.mean([n_sel[i % nsets] for i in range(0, args.steps + SAMPLE_EXTRA, TIME_EVERY)]))
    else:
        nsel_mean = nsel_gu = float(np.mean(n_sel))
    layer_bytes = nsel_mean * expert_bytes + wl.E * wl.d * 2 + wl.E * 4 + 2 * x_bytes
    step_bytes = layer_bytes * nlay
    step_flops = 2.0 * P * 3 * wl.d * wl.I * nlay
    gu_unit_bytes = mxfp4_bytes(2 * wl.I, wl.d) + 4 * 2 * wl.I
    gu_bytes = nsel_gu * gu_unit_bytes + x_bytes
    gu_flops = 2.0 * P * wl.d * 2 * wl.I
    traffic = read_traffic("gateup_gemm", wl.name) if args.act == "exact" else None
    hbm_kernel_rm = gu_bytes / (gu_us_rm * 1e-6)
    hbm_kernel = gu_bytes / (gu_us * 1e-6)
    mfma_kernel = gu_flops / (gu_us * 1e-6)
    if bound == "hbm":
        roof = {"bound": "hbm", "achieved": hbm_kernel / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                "frac": hbm_kernel / HBM_PEAK, "traffic": traffic, "kernel": "gateup_gemm", "kernel_us": gu_us,
                "algorithmic_bytes_per_launch": gu_bytes}
    else:
        roof = {"bound": "mfma", "achieved": mfma_kernel / 1e12, "peak": MFMA_FP6_FP4_PEAK / 1e12,
                "unit": "TFLOP/s", "frac": mfma_kernel / MFMA_FP6_FP4_PEAK, "traffic": traffic,
                "kernel": "gateup_gemm", "kernel_us": gu_us, "algorithmic_flops_per_launch": gu_flops,
                # every algorithmic 16x16x128 step issues three MFMAs (one per FP6 term)
                "issued_mfma_frac": 3 * mfma_kernel / MFMA_FP6_FP4_PEAK,
                "hbm_frac_of_weights": hbm_kernel / HBM_PEAK}

    rec = {
        "value": tok_s,
        "unit": "tokens/s",
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "config": {
            "workload": wl.name, "T": wl.T, "d": wl.d, "I": wl.I, "E": wl.E, "k": wl.k, "layers": nlay,
            "routing": wl.routing, "weight_sets": nsets if nlay == 1 else 1,
            "experts_hit_mean": nsel_mean,
            "hbm_bytes_per_step": step_bytes, "hbm_GBps": step_bytes / (ms_step * 1e-3) / 1e9,
            "hbm_frac": step_bytes / (ms_step * 1e-3) / HBM_PEAK,
            "flops_per_step": step_flops, "TFLOPs": step_flops / (ms_step * 1e-3) / 1e12,
            "mxfp4_mfma_frac": step_flops / (ms_step * 1e-3) / MFMA_FP6_FP4_PEAK,
            "kernel_us": {k: (v[0] / v[1] * 1e3 if v[1] else None) for k, v in kt.items()},
            "parallelism": "single-gpu",
            "activations": {"exact": "three-term MX6x3 (each value to about 2^-13 of its 32-block maximum)",
                            "mxfp6": "mxfp6 (activation-quantised fast mode)",
                            "mx6x2": "two-term MX6 (MOE_LAYER_MX6X2; each value within 1/225 of its 32-block "
                                     "maximum)"}[args.act],
            "weight_layout": "packed MXFP4 (moe_pack_weights once per weight set before timing; "
                             "MOE_LAYER_PACKED); the same bytes as the stored format",
            "rowmajor": {
                "weight_layout": "row-major MXFP4 as stored (moe_layer_forward / moe_stack_forward)",
                "ms_per_step": ms_rm, "value": wl.T / (ms_rm * 1e-3),
                "gateup_gemm_us": gu_us_rm,
                "kernel_us": {k: (v[0] / v[1] * 1e3 if v[1] else None) for k, v in kt_rm.items()},
                "gateup_roofline_frac": (hbm_kernel_rm / HBM_PEAK) if bound == "hbm"
                                        else gu_flops / (gu_us_rm * 1e-6) / MFMA_FP6_FP4_PEAK,
            },
        },
        "roofline": roof,
        "cpu_baseline": None,
    }
    # free this leg's device memory before the next leg
    sets.clear()
    psets.clear()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if want_cpu and host0 is not None:
        rec["cpu_baseline"] = cpu_baseline(wl, host0, args.cpu_budget, args.act)
        log(f"cpu baseline: {rec['cpu_baseline']}")
    return rec


def attn_work(wl):
    """Algorithmic work of one attention call: (FLOPs, HBM bytes).  FLOPs
    count 2 per multiply-add of q.k and of p.v over the keys each query sees;
    bytes read q and every key/value row some query sees once, and write out."""
    import numpy as np
    pos = wl.q_pos0 + np.arange(wl.Tq)
    lo = np.maximum(0, pos - wl.window + 1) if wl.window > 0 else np.zeros_like(pos)
    seen = int(np.sum(pos - lo + 1))
    flops = 4.0 * wl.D * wl.Hq * seen * wl.B
    keys = int(pos[-1] - lo[0] + 1)
    nbytes = wl.B * (2 * wl.Tq * wl.Hq * wl.D * 2 + 2 * keys * wl.Hkv * wl.D * 2)
    return flops, float(nbytes)


def run_attn_leg(wl, args, torch, moe, want_cpu):
    """Times one attention workload (one kernel per call); the roofline is
    bf16 MFMA for dense prefill, HBM otherwise."""
    import numpy as np
    from moe_inputs import synth
    flops, nbytes = attn_work(wl)
    per_set = wl.B * (wl.Tq * wl.Hq + 2 * wl.S * wl.Hkv) * wl.D * 2
    nsets = max(1, min(4, int(np.ceil(1.1e9 / per_set))))
    log(f"attention workload {wl.name}: B={wl.B} Tq={wl.Tq} S={wl.S} q_pos0={wl.q_pos0} Hq={wl.Hq} "
        f"Hkv={wl.Hkv} D={wl.D} window={wl.window} sets={nsets}")
    sets, host0 = [], None
    for i in range(nsets):
        q, k, v, sinks = synth.gen_attention(wl.seed + 1000 * i, wl.B, wl.Tq, wl.S, wl.Hq, wl.Hkv, wl.D)
        if i == 0 and want_cpu:
            host0 = (q, k, v, sinks)
        dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to("cuda:0")
        sets.append((dev(q), dev(k), dev(v), torch.from_numpy(sinks).to("cuda:0"), torch.empty(
            (wl.B, wl.Tq, wl.Hq, wl.D), dtype=torch.bfloat16, device="cuda:0")))
    torch.cuda.synchronize()

    def step(i):
        q, k, v, s, o = sets[i % nsets]
        moe.moe_attn_forward(q, k, v, s, q_pos0=wl.q_pos0, window=wl.window, out=o)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for i in range(args.steps):
        step(i)
    ev1.record()
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) / args.steps * 1e3
    log(f"timed {args.steps} calls: {us:.1f} us/call")
    dense_prefill = wl.window == 0 and wl.Tq > 1
    if dense_prefill:
        roof = {"bound": "mfma", "achieved": flops / (us * 1e-6) / 1e12, "peak": BF16_MFMA_PEAK / 1e12,
                "unit": "TFLOP/s", "frac": flops / (us * 1e-6) / BF16_MFMA_PEAK, "traffic": None,
                "kernel": "attn_kernel", "kernel_us": us, "algorithmic_flops_per_launch": flops}
    else:
        roof = {"bound": "hbm", "achieved": nbytes / (us * 1e-6) / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                "frac": nbytes / (us * 1e-6) / HBM_PEAK, "traffic": None, "kernel": "attn_kernel",
                "kernel_us": us, "algorithmic_bytes_per_launch": nbytes}
    rec = {"value": wl.B * wl.Tq / (us * 1e-6), "unit": "tokens/s", "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": us * 1e-3,
           "config": {"workload": wl.name, "B": wl.B, "Tq": wl.Tq, "S": wl.S, "q_pos0": wl.q_pos0, "Hq": wl.Hq,
                      "Hkv": wl.Hkv, "D": wl.D, "window": wl.window, "sets": nsets,
                      "flops_per_call": flops, "hbm_bytes_per_call": nbytes,
                      "note": "one kernel per call; the time is HIP events around the timed calls"},
           "roofline": roof, "cpu_baseline": None}
    sets.clear()
    torch.cuda.empty_cache()
    if want_cpu and host0 is not None:
        rec["cpu_baseline"] = attn_cpu_baseline(wl, host0, args.cpu_budget / 2)
        log(f"cpu baseline: {rec['cpu_baseline']}")
    return rec


def attn_cpu_baseline(wl, host, budget_s):
    """The fp64 attention oracle on query tokens taken from the end of the
    batch (all heads of each), repeated until about budget_s is spent."""
    from oracle import attention_oracle as A
    from oracle.moe_oracle import bf16_bits_to_f64
    q, k, v, sinks = host
    b = wl.B - 1
    qf = bf16_bits_to_f64(q[b:b + 1])
    kf, vf = bf16_bits_to_f64(k[b:b + 1]), bf16_bits_to_f64(v[b:b + 1])
    s64 = sinks.astype("float64")
    model, ncpu = host_cpu()
    done, total, i = 0, 0.0, wl.Tq - 1
    while total < budget_s and done < wl.Tq:
        rows = [(0, i, h) for h in range(wl.Hq)]
        t0 = time.perf_counter()
        A.attention_rows(qf, kf, vf, s64, wl.q_pos0, wl.window, rows)
        total += time.perf_counter() - t0
        done += 1
        i = (i - 1) % wl.Tq
    return {"value": done / total, "unit": "tokens/s", "cores": 1, "kind": "oracle", "cpu_model": model,
            "nproc": ncpu, "sample": f"{done} query tokens (all {wl.Hq} heads) from the end of sequence {b}, "
                                     f"fp64 numpy oracle row by row, {total:.1f} s"}


def main():
    from moe_inputs.workloads import ATTN_WORKLOADS, WORKLOADS
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None, choices=sorted(WORKLOADS) + sorted(ATTN_WORKLOADS),
                    help="one workload as the headline (default: every leg of the metric)")
    ap.add_argument("--sets", type=int, default=0, help="weight sets to rotate over (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=16.0, help="seconds of oracle time per leg")
    ap.add_argument("--act", default="exact", choices=["exact", "mxfp6", "mx6x2"],
                    help="expert-GEMM activations: exact (three FP6 terms), mxfp6 (the "
                         "activation-quantised fast mode, one term) or mx6x2 (the two-term option)")
    ap.add_argument("--no-attention", action="store_true", help="leave out the attention legs of the default run")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one 256 MiB bitwise_not kernel (reads and writes 256 MiB: "
                         "the reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the MoE layer here is built and measured on a single MI355X, "
              f"and no multi-GPU path exists (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be at least 1 and --warmup at least 0", file=sys.stderr)
        sys.exit(2)
    if args.workload in ATTN_WORKLOADS:
        legs = [(args.workload, "attn")]
    else:
        legs = LEGS if args.workload is None else [(args.workload, None)]
        if args.workload is None and not args.no_attention:
            legs = [(n, "attn") for n in ATTN_LEGS] + legs
    if args.act != "exact" and any(b != "attn" and WORKLOADS[n].layers > 1 for n, b in legs):
        print("the one- and two-term activation options have single-layer entry points only; pick a "
              "single-layer --workload", file=sys.stderr)
        sys.exit(2)

    import torch
    import sparse_moe_transformer_softmax_amd as moe

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    moe.lib()
    if args.copy_calibration:
        a = torch.empty(64 << 20, dtype=torch.int32, device="cuda:0").fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        torch.bitwise_not(a, out=b)
        torch.cuda.synchronize()
        del a, b

    recs = {}
    for name, bound in legs:
        if bound == "attn":
            recs[name] = run_attn_leg(ATTN_WORKLOADS[name], args, torch, moe, want_cpu=not args.no_cpu_baseline)
            continue
        wl = WORKLOADS[name]
        if bound is None:
            bound = "hbm" if wl.T * wl.k <= 32 * wl.E or wl.layers > 1 else "mfma"
        recs[name] = run_leg(wl, bound, args, torch, moe, want_cpu=not args.no_cpu_baseline)

    head_name = legs[-1][0]
    head = recs[head_name]
    line = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if legs[-1][1] == "attn" else "mxfp4",
        "data": "synthetic",
        "config": head["config"],
        "roofline": head["roofline"],
        "cpu_baseline": head["cpu_baseline"],
    }
    if len(legs) > 1:
        line["legs"] = {n: recs[n] for n, _ in legs[:-1]}
        if not args.no_cpu_baseline:
            line["cpu_one_thread"] = one_thread_rates(4.0)
            log(f"oracle on one thread: {line['cpu_one_thread']}")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python
"""Benchmark of the 2-bit routed-expert MoE layer on one MI355X.

Metric: MoE-layer tokens/s plus achieved HBM GB/s on the quantized expert bytes,
for decode and prefill.  A step is one pass of the whole layer (routing,
bucketing, routed Q2 experts, bf16 shared expert, combine; for the residual
stack also RMSNorm and the residual add) over one batch of synthetic input with
all weights resident in HBM.  Decode steps rotate over several distinct layers
of the same shape (as a model's layer stack does), so each step streams its
weights from HBM rather than from the 256 MB last-level cache.

Steps are timed as HIP graph replays by default (one captured graph holds one
pass over the rotated layers, or one step; exactly K steps are replayed), which
removes the host-side launch cost of the ~15 kernels of a decode step; the dominant
routed kernel's duration comes from HIP events that its own launch records (start and
end of the kernel's dispatch) in a separate eager loop of the same K steps, which is
also reported (eager_ms_per_step).  --graph 0 times the eager loop only.

Prints ONE JSON line.  Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
MFMA_INT8_PEAK_TOPS = 5000.0
PCIE_PEAK_GBS = 64.0            # PCIe 5.0 x16, one direction, nominal
EXPERT_BYTES_FULL = 14_450_688
METRIC = "MoE-layer tokens/s + achieved HBM GB/s (2-bit experts), decode and prefill"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=48)
    ap.add_argument("--workload", default="decode1")
    ap.add_argument("--extra", default="decode32_zipf,prefill2048,stack40_t64_zipf,verify96_zipf,verify96_zipf:bi,"
                                       "stack40_q2q4,decode32_zipf:q8,prefill2048:q8,prefill2048_q4,decode32_zipf:cache,"
                                       "decode32_zipf:cache_admit",
                    help="comma-separated extra workloads reported in the same line ('' for none)")
    ap.add_argument("--rotate", type=int, default=8, help="distinct layers cycled by decode steps")
    ap.add_argument("--cpu-baseline", type=int, default=1)
    ap.add_argument("--graph", type=int, default=1, help="time steps as HIP graph replays")
    ap.add_argument("--ceilings", type=int, default=1, help="measure copy and bf16 GEMM ceilings")
    ap.add_argument("--warm", type=int, default=1,
                    help="also time the headline workload on one layer (weights largely cache-resident)")
    ap.add_argument("--calibrate-copy", type=int, default=0,
                    help="also run a plain 1 GiB device copy (reference for HBM byte counters)")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def layer_bytes(wl, touched):
    """Algorithmic HBM bytes of one layer step: touched Q2 experts, bf16 shared
    expert, fp32 router, activations in (bf16/fp32) and output out (fp32)."""
    act_in = 4 if (wl.act == "f32" or wl.rmsnorm) else 2
    b = touched * wl.expert_bytes + 3 * wl.shared_inter * wl.hidden * 2 \
        + wl.n_experts * wl.hidden * 4 + wl.tokens * wl.hidden * (act_in + 4)
    if wl.rmsnorm:
        b += wl.tokens * wl.hidden * 4      # residual read-modify-write
    return b


def library_source(text):
    """A kernel source as libmoe_q2.so compiles it: without the per-work-group timeline
    marks, which exist only in the timeline build (every line naming one contains
    "MQ_TL"; the device array and its accessors sit in one "#ifdef MQ_WG_TIMELINE"
    block; the include of timeline.h)."""
    out, depth = [], 0
    for line in text.splitlines(keepends=True):
        st = line.strip()
        if depth:
            if st.startswith("#if"):
                depth += 1
            elif st.startswith("#endif"):
                depth -= 1
            continue
        if st == "#ifdef MQ_WG_TIMELINE":
            depth = 1
        elif "MQ_TL" not in line and st != '#include "timeline.h"':
            out.append(line)
    return "".join(out)


def traffic_record(kernel):
    """HBM traffic per launch from committed rocprofv3 counter runs, valid only while
    the kernel source, as the library compiles it, is unchanged (sha256 recorded with
    the counters)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(kernel)
    if not rec:
        return None
    src = os.path.join(ROOT, rec["source"])
    sha = hashlib.sha256(library_source(open(src).read()).encode()).hexdigest()
    if sha != rec["source_sha256"]:
        return None
    return rec


# Row options: "name:q8" (Q8 activations), "name:bi" (batch-invariant mode).
ROW_FLAGS = {"": 0, "q8": 128, "bi": 64}


def matrix_bytes(wl, layer):
    """(gate + up, down) bytes of one routed expert of a layer (formats per layer)."""
    nb = wl.hidden * wl.inter // 256
    gu4, dn4 = wl.q4_at(layer)
    return 2 * nb * (148 if gu4 else 84), nb * (148 if dn4 else 84)


def run_workload(spec, steps, warmup, rotate, graph=True):
    import torch
    import bit_quantized_routed_amd as mq
    from bit_quantized_routed_amd import workload as dw
    from synth import workloads as W

    name, _, opt = spec.partition(":")
    wl = W.WORKLOADS[name]
    L = wl.layers if wl.layers > 1 else rotate
    t0 = time.time()
    tmp = torch.empty(wl.hidden * wl.inter, dtype=torch.float32, device="cuda")
    layers = [dw.DeviceLayer(wl, layer=l, tmp=tmp) for l in range(L)]
    del tmp
    torch.cuda.synchronize()
    log("[bench] %s: %d layer(s) generated in %.1fs" % (spec, L, time.time() - t0))
    T, K, E = wl.tokens, wl.topk, wl.n_experts
    flags = (mq.RESIDUAL_ADD if wl.rmsnorm else 0) | ROW_FLAGS[opt]
    shapes = [layer.shape(flags) for layer in layers]        # per layer: the weight formats
    shape = shapes[0]
    ws = torch.empty(max(mq.workspace_size(sh, T, K) for sh in shapes), dtype=torch.uint8, device="cuda")
    x = dw.activations(wl)
    out = x if wl.rmsnorm else torch.empty((T, wl.hidden), dtype=torch.float32, device="cuda")
    counts = [torch.zeros(E, dtype=torch.int32, device="cuda") for _ in range(L)]
    stack = wl.layers > 1            # one step = the whole residual stack

    def one_pass(i, events=None):
        l = i % L
        tr = {"counts": counts[l]}
        if events is not None:
            tr["events"] = events
        mq.forward(x, layers[l].router_w, layers[l].experts, layers[l].shared_w, K, out, shapes[l], T,
                   router_b=layers[l].router_b, workspace=ws, trace=tr)

    def step(i, evs=None):
        if stack:
            for l in range(L):
                one_pass(l, None if evs is None else evs[l])
        else:
            one_pass(i, evs)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    n_ev = L if stack else 1
    # untimed instrumented pass: per-phase breakdown (every phase bracketed)
    prof_steps = min(steps, 5)
    phase = {p: [] for p in mq.PHASES}
    for i in range(prof_steps):
        es = [mq.EventSet() for _ in range(n_ev)]
        step(i, es if stack else es[0])
        for e in es:
            for p, v in e.elapsed().items():
                phase[p].append(v)
            e.close()
    phase_ms = {p: float(np.mean(v)) for p, v in phase.items() if v}
    # roofline kernel: the larger of the two routed-expert kernels (single launches)
    dom = max(("gate_up", "down"), key=lambda p: phase_ms.get(p, 0.0))
    # timed region: only the dominant kernel's phase is bracketed by events
    evsets = [[mq.EventSet(phases=[dom]) for _ in range(n_ev)] for _ in range(steps)]
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(steps):
        step(i, evsets[i] if stack else evsets[i][0])
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    ms_per_step = (t2 - t1) * 1e3 / steps
    dom_ms = []
    for es in evsets:
        for e in es:
            dom_ms.append(e.elapsed()[dom])
            e.close()
    dom_avg = float(np.mean(dom_ms))
    eager_ms = ms_per_step
    pct = None
    launch = "eager"
    if graph:
        # One captured graph holds one pass over the rotated layers (L consecutive
        # steps; the whole stack for the residual stack, which is one step), plus one
        # graph of the first steps % L steps: full passes are replayed steps // L times,
        # then the remainder once -- exactly `steps` steps for any step count, one host
        # launch per pass.
        G = 1 if stack else L
        n_full, rem = steps // G, steps % G
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            for i in range(G):
                step(i)
        torch.cuda.current_stream().wait_stream(cap)
        torch.cuda.synchronize()
        full = torch.cuda.CUDAGraph()
        with torch.cuda.graph(full):
            for i in range(G):
                step(i)
        part = None
        if rem:
            part = torch.cuda.CUDAGraph()
            with torch.cuda.graph(part):
                for i in range(rem):
                    step(i)
        for r in range(max(1, warmup // G)):
            full.replay()
        if part is not None:            # its first launch (graph upload) stays out of the timing
            part.replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for r in range(n_full):
            full.replay()
        if part is not None:
            part.replay()
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        ms_per_step = (t2 - t1) * 1e3 / steps
        launch = "hip_graph, %d step(s) per replay" % G
        # spread of the step time: a separate pass of event-bracketed full replays
        n_pct = max(10, min(60, max(n_full, 1)))
        pev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n_pct)]
        for r in range(n_pct):
            pev[r][0].record()
            full.replay()
            pev[r][1].record()
        torch.cuda.synchronize()
        per_step = [a.elapsed_time(b) / G for a, b in pev]
        pct = {"p10": float(np.percentile(per_step, 10)), "p50": float(np.percentile(per_step, 50)),
               "p90": float(np.percentile(per_step, 90)), "replays": n_pct}
        del full, part
    touched = [int((c > 0).sum().item()) for c in counts]
    d_mean = float(np.mean(touched))
    passes = L if stack else 1
    tokens_per_step = T * (1 if not stack else 1)
    mb = [matrix_bytes(wl, l) for l in range(L)]
    # routed bytes per pass, averaged over the rotated (or stacked) layers
    routed_gu = float(np.mean([t * m[0] for t, m in zip(touched, mb)]))
    routed_dn = float(np.mean([t * m[1] for t, m in zip(touched, mb)]))
    bytes_per_pass = layer_bytes(wl, 0) + routed_gu + routed_dn
    res = {
        "workload": spec, "tokens": T, "layers_in_step": passes, "layers_resident": L,
        "flags": flags,
        "ms_per_step": ms_per_step, "eager_ms_per_step": eager_ms, "launch": launch,
        "tokens_per_s": tokens_per_step / (ms_per_step * 1e-3),
        "layer_tokens_per_s": T * passes / (ms_per_step * 1e-3),
        "touched_experts_mean": d_mean, "touched_experts_per_layer": touched,
        "algorithmic_bytes_per_pass": bytes_per_pass,
        "hbm_gbs": bytes_per_pass * passes / (ms_per_step * 1e-3) / 1e9,
        "phases_ms_per_pass": phase_ms,
        "ms_per_step_percentiles": pct,
        "phases_note": "separate instrumented pass; gate_up and down are the kernels' own start-to-end times, the other phases are bracketed by events (~4 us of overhead each)",
    }
    # dominant kernel roofline (duration from the timed region's events); on the
    # matrix-core decode path with a bf16 layer input the routed launches also
    # stream the shared expert's gate/up and down rows
    gu_bytes = routed_gu
    dn_bytes = routed_dn
    if T < 256 and wl.shared_inter and (wl.act == "bf16" or wl.rmsnorm):
        gu_bytes += 2 * wl.shared_inter * wl.hidden * 2
        dn_bytes += wl.shared_inter * wl.hidden * 2
    launch_bytes = {"gate_up": gu_bytes + T * wl.hidden * 2.5 + T * K * wl.inter * 4,
                    "down": dn_bytes + T * K * wl.inter * 2.5 + T * K * wl.hidden * 4,
                    "shared": 3 * wl.shared_inter * wl.hidden * 2}
    kbytes = launch_bytes.get(dom)
    prefill = mq.describe(shape, T, K)["path"] == mq.PATH_PREFILL
    if prefill:
        # useful MACs x 2 against the dense MFMA peak of the arithmetic: the default path
        # issues two int8 MACs per useful MAC on units twice the bf16 rate (the same
        # fraction of the bf16 peak as of the int8 peak); Q8 issues one int8 MAC per
        # useful MAC, against the int8 peak
        q8 = bool(flags & mq.ACT_Q8)
        peak = MFMA_INT8_PEAK_TOPS if q8 else MFMA_BF16_PEAK_TFLOPS
        kflops = {"gate_up": T * K * 2 * wl.inter * wl.hidden * 2,
                  "down": T * K * wl.hidden * wl.inter * 2,
                  "shared": T * 3 * wl.shared_inter * wl.hidden * 2}[dom]
        ach = kflops / (dom_avg * 1e-3) / 1e12
        res["roofline"] = {"bound": "mfma", "kernel": dom, "achieved": round(ach, 1),
                           "peak": peak, "unit": "TOP/s (int8)" if q8 else "TFLOP/s",
                           "frac": round(ach / peak, 4), "traffic": None,
                           "algorithmic_flops_per_launch": kflops, "avg_launch_ms": dom_avg}
        res["useful_tflops"] = (T * K * 3 * wl.inter * wl.hidden * 2 +
                                T * 3 * wl.shared_inter * wl.hidden * 2) / (ms_per_step * 1e-3) / 1e12
    elif kbytes is not None and dom_avg > 0:
        ach = kbytes / (dom_avg * 1e-3) / 1e9
        tr = traffic_record("%s/%s" % (spec, dom))
        res["roofline"] = {"bound": "hbm", "kernel": dom, "achieved": round(ach, 1),
                           "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                           "traffic": None if tr is None else tr.get("bytes_per_launch"),
                           "algorithmic_bytes_per_launch": kbytes,
                           "algorithmic_bytes_by_launch": {k: launch_bytes[k] for k in ("gate_up", "down")},
                           "avg_launch_ms": dom_avg}
    # one more untimed forward of layer 0 with its routing traced, kept for the parity
    # check against the oracle's outputs of the CPU baseline (first tokens only)
    npar = min(T, 8)
    x0 = dw.activations(wl)
    o0 = x0.clone() if wl.rmsnorm else torch.zeros((T, wl.hidden), dtype=torch.float32, device="cuda")
    ti = torch.full((T, K), -1, dtype=torch.int32, device="cuda")
    mq.forward(x0, layers[0].router_w, layers[0].experts, layers[0].shared_w, K, o0, shape, T,
               router_b=layers[0].router_b, workspace=ws, trace={"topk_idx": ti})
    torch.cuda.synchronize()
    res["_gpu_first_tokens"] = {"out": o0[:npar].cpu().numpy().astype(np.float64),
                                "idx": ti[:npar].cpu().numpy()}
    del layers, ws, x0, o0
    torch.cuda.empty_cache()
    return res


def run_cached(spec, steps, warmup, budget=0.5, n_batches=64):
    """A layer whose routed experts live in pinned host memory behind an HBM expert
    cache of `budget` x E slots (moe_q2_forward_cached), fed a stream of distinct
    micro-batches (n_batches batches of the workload's token count, cycled), so the
    routing -- and with it the hits and misses -- changes from step to step as in a
    serving loop.  Eager timing; the same stream through the resident layer is timed
    alongside.  Reported: step time, hit rate, misses per step (copied into slots, or
    read straight from host memory when the free slots run out) and the host-link
    rate of the bytes brought over per step."""
    import torch
    import bit_quantized_routed_amd as mq
    from bit_quantized_routed_amd import workload as dw
    from synth import workloads as W

    name, _, opt = spec.partition(":")
    policy = mq.CACHE_LRU_ADMIT if opt == "cache_admit" else mq.CACHE_LRU
    wl = W.WORKLOADS[name]
    T, K, E = wl.tokens, wl.topk, wl.n_experts
    dl = dw.DeviceLayer(wl)
    eb = wl.expert_bytes
    t0 = time.time()
    host = torch.empty(E * eb, dtype=torch.uint8, pin_memory=True)
    host.copy_(dl.experts)
    torch.cuda.synchronize()
    log("[bench] %s: %.1f GB of experts in pinned host memory (%.1fs)" % (spec, E * eb / 1e9, time.time() - t0))
    n_slots = int(E * budget)
    slots = torch.empty(n_slots * eb, dtype=torch.uint8, device="cuda")
    state = torch.empty(mq.cache_state_bytes(n_slots, E) // 4, dtype=torch.int32, device="cuda")
    cache = mq.make_cache(slots, eb, n_slots, E, state, policy=policy)
    mq.cache_reset(cache)
    shape = dl.shape(0)
    ws = dw.workspace(shape, T, K)
    xs = dw.activations(wl, tokens=T * n_batches)
    out = torch.empty((T, wl.hidden), dtype=torch.float32, device="cuda")

    def cached(i):
        b = i % n_batches
        mq.forward_cached(xs[b * T:(b + 1) * T], dl.router_w, host, 0, cache, dl.shared_w, K, out, shape, T,
                          router_b=dl.router_b, workspace=ws)

    def resident(i):
        b = i % n_batches
        mq.forward(xs[b * T:(b + 1) * T], dl.router_w, dl.experts, dl.shared_w, K, out, shape, T,
                   router_b=dl.router_b, workspace=ws)

    def timed(fn, first):
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for i in range(first, first + steps):
            fn(i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t1) * 1e3 / steps

    for i in range(warmup):
        cached(i)
    st0 = state[:8].cpu().numpy().astype(np.int64)
    ms = timed(cached, warmup)
    st1 = state[:8].cpu().numpy().astype(np.int64)
    for i in range(warmup):
        resident(i)
    ms_res = timed(resident, warmup)
    hits, misses, unc = (st1[1] - st0[1]) / steps, (st1[2] - st0[2]) / steps, (st1[6] - st0[6]) / steps
    host_bytes = misses * eb            # copied once, or read once by the routed kernels
    res = {"workload": spec, "tokens": T, "budget_experts": n_slots, "budget_bytes": n_slots * eb,
           "experts_per_layer": E, "launch": "eager", "ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3),
           "resident_ms_per_step": ms_res, "hit_rate": hits / max(hits + misses, 1e-9),
           "touched_per_step": hits + misses, "misses_per_step": misses, "uncached_per_step": unc,
           "host_bytes_per_step": host_bytes, "host_link_gbs": host_bytes / (ms * 1e-3) / 1e9,
           "host_link_peak_gbs": PCIE_PEAK_GBS,
           "policy": "lru with frequency admission" if policy == mq.CACHE_LRU_ADMIT else "lru",
           "note": "distinct %d-token batches cycled (%d), experts homed in pinned host memory, %d of %d "
                   "experts' slots in HBM" % (T, n_batches, n_slots, E)}
    del dl, host, slots, xs, ws
    torch.cuda.empty_cache()
    return res


def W_layers(spec):
    from synth import workloads as W
    return W.WORKLOADS[spec.partition(":")[0]].layers


def measured_ceilings():
    """Context for the roofline fractions, measured on the same GPU: a 2 GiB
    device-to-device copy (GB/s counting read + write) and a bf16 8192^3 matrix
    product through torch's BLAS (TFLOP/s); medians of 10 timed repetitions."""
    import torch

    def timed(fn, n=10):
        fn()
        torch.cuda.synchronize()
        ms = []
        for _ in range(n):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ms.append(a.elapsed_time(b))
        return float(np.median(ms))

    nb = 1 << 31
    src = torch.ones(nb // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    copy_ms = timed(lambda: dst.copy_(src))
    del src, dst
    n = 8192
    a = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    b = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    gemm_ms = timed(lambda: torch.matmul(a, b))
    del a, b
    torch.cuda.empty_cache()
    return {"copy_gbs": round(2 * nb / (copy_ms * 1e-3) / 1e9, 1),
            "gemm_bf16_tflops": round(2 * n ** 3 / (gemm_ms * 1e-3) / 1e12, 1),
            "note": "2 GiB device copy (read + write bytes) and bf16 8192^3 torch.matmul, medians of 10"}


# How the oracle is timed per workload: tokens per oracle call, runs per token
# (median), the minimum oracle time of the headline sample, and the layer count a
# one-layer time is scaled by (the residual stack: one layer timed, x40, labelled).
CPU_PROTOCOL = {
    "tiny": dict(tokens_per_call=4, max_calls=1, runs=3),
    "decode1": dict(tokens_per_call=1, max_calls=8, runs=1, min_seconds=10.0),
    "decode32_zipf": dict(tokens_per_call=1, max_calls=1, runs=3),
    "prefill2048": dict(tokens_per_call=1, max_calls=1, runs=1),
    "stack40_t64_zipf": dict(tokens_per_call=1, max_calls=1, runs=1, scale_layers=40),
}


def cpu_baseline(name, gpu=None):
    """The oracle, untuned, on the host cores for a bounded sample of the workload
    (CPU_PROTOCOL): the layer (for the residual stack: RMSNorm, layer 0, residual add)
    on the workload's first tokens, the routed experts of each call encoded to Q2 bytes
    beforehand, untimed (input preparation); tokens/s from the summed per-call medians.
    With `gpu` (the GPU's outputs and routing of the same first tokens of layer 0),
    also a parity summary: per-token infinity-norm relative error, near-tie tokens,
    routing-set mismatches outside the near-tie window."""
    from oracle import moe
    from tests.oracle_inputs import HostLayer
    from synth import workloads as W
    try:
        from threadpoolctl import threadpool_info
        thr = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        thr = 1
    wl = W.WORKLOADS[name]
    pr = CPU_PROTOCOL.get(name, dict(tokens_per_call=1, max_calls=1, runs=1))
    tpc, runs, scale = pr["tokens_per_call"], pr["runs"], pr.get("scale_layers", 1)
    n_max = tpc * pr["max_calls"]
    hl = HostLayer(wl, 0)
    x_all, _ = W.activations(wl, tokens=max(n_max, wl.tokens))
    xin = moe.rmsnorm_bf16(x_all, wl.rms_eps) if wl.rmsnorm else x_all
    idx, _, logits, margin = moe.route(xin, hl.router_w, hl.router_b, wl.topk)
    total, n, refs = 0.0, 0, []
    while n < n_max and total < pr.get("min_seconds", 0.0) or n == 0:
        rows = slice(n, n + tpc)
        for e in np.unique(idx[rows]):
            hl.expert_bytes(int(e))          # untimed: input preparation
        times = []
        for _ in range(runs):
            t = time.perf_counter()
            if wl.rmsnorm:
                ref, _ = moe.stack(x_all[rows], [hl.oracle_layer()], wl.topk, wl.hidden, wl.inter, wl.rms_eps)
            else:
                ref, _ = moe.layer(x_all[rows], hl.router_w, hl.router_b, hl.expert_bytes, hl.shared, wl.topk,
                                   wl.hidden, wl.inter)
            times.append(time.perf_counter() - t)
        total += float(np.median(times))
        refs.append(ref)
        n += tpc
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), None)
    except OSError:
        pass
    res = {"value": round(n / (total * scale), 4), "unit": "tokens/s" if scale == 1 else "tokens/s per %d-layer step" % scale,
           "cores": int(thr), "affinity_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu_model,
           "kind": "oracle",
           "sample": "first %d token(s) of layer 0 of %s, %d token(s) per oracle call, median of %d run(s) per "
                     "call (routing, dequantisation of the touched experts, fp64 FFNs, shared expert, combine%s); "
                     "%.2f s of oracle time%s" % (n, name, tpc, runs, ", RMSNorm and residual" if wl.rmsnorm else "",
                                                  total, ("; one layer timed, x%d layers: extrapolated" % scale)
                                                  if scale > 1 else "")}
    if gpu is not None:
        ref = np.concatenate(refs)[:len(gpu["out"])]
        m = min(len(ref), len(gpu["out"]))
        near = margin[:m] < 1e-4
        mism = sum(1 for t in range(m) if not near[t] and set(gpu["idx"][t].tolist()) != set(idx[t].tolist()))
        num = np.abs(gpu["out"][:m] - ref[:m]).max(axis=1)
        den = np.abs(ref[:m]).max(axis=1)
        err = (num / den)[~near]
        res["parity"] = {"tokens_compared": int((~near).sum()), "near_tie_excluded": int(near.sum()),
                         "routing_mismatches": int(mism), "max_rel_err": float(err.max()) if err.size else None,
                         "what": "GPU layer 0 outputs of the same first tokens against the oracle's"}
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: the layer runs on one GPU; --gpus %d is not supported" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(2)
    head = run_workload(args.workload, args.steps, args.warmup, args.rotate, bool(args.graph))
    extras = {}
    for name in [n for n in args.extra.split(",") if n and n != args.workload]:
        if name.endswith(":cache") or name.endswith(":cache_admit"):
            extras[name] = run_cached(name, args.steps, args.warmup)
        else:
            extras[name] = run_workload(name, args.steps, args.warmup, args.rotate, bool(args.graph))
    if args.calibrate_copy:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1.0)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    warm = None
    if args.warm and W_layers(args.workload) == 1:
        wr = run_workload(args.workload, min(args.steps, 200), args.warmup, 1, bool(args.graph))
        warm = {"ms_per_step": round(wr["ms_per_step"], 5), "tokens_per_s": round(wr["tokens_per_s"], 2),
                "note": "the same layer every step (its 211 MB largely held by the 256 MB MALL); "
                        "labelled warm, not the headline"}
    ceil = measured_ceilings() if args.ceilings else None
    cpu = None
    if args.cpu_baseline:
        cpu = cpu_baseline(args.workload.partition(":")[0], head.pop("_gpu_first_tokens", None))
        for k, v in extras.items():
            if k in CPU_PROTOCOL:           # the oracle's time does not depend on the row options
                v["cpu_baseline"] = cpu_baseline(k, v.pop("_gpu_first_tokens", None))
    head.pop("_gpu_first_tokens", None)
    for v in extras.values():
        v.pop("_gpu_first_tokens", None)
    from synth import workloads as W
    wl = W.WORKLOADS[args.workload.partition(":")[0]]
    line = {
        "metric": METRIC, "value": round(head["tokens_per_s"], 2), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "i8mfma+fp32", "data": "synthetic",
        "dtype_note": "routed experts: exact int8 q*sc codes x int8 digits of 15-bit activations on the "
                      "integer matrix cores (int32 sums per block), d/dmin folded in fp32; bf16 shared expert "
                      "on bf16 MFMA with fp32 accumulation; fp32 router; fp32 output",
        "config": {"workload": args.workload, "tokens": wl.tokens, "hidden": wl.hidden,
                   "n_experts": wl.n_experts, "topk": wl.topk, "inter": wl.inter,
                   "shared_inter": wl.shared_inter, "weights": "q2 routed (84 B/256), bf16 shared, fp32 router",
                   "layers_rotated": head["layers_resident"], "launch": head["launch"],
                   "eager_ms_per_step": round(head["eager_ms_per_step"], 5),
                   "touched_experts_mean": head["touched_experts_mean"]},
        "hbm_gbs": round(head["hbm_gbs"], 1),
        "roofline": head.get("roofline"),
        "ms_per_step_percentiles": head.get("ms_per_step_percentiles"),
        "measured_ceilings": ceil,
        "warm": warm,
        "cpu_baseline": cpu,
        "phases_ms": {k: round(v, 5) for k, v in head["phases_ms_per_pass"].items()},
        "parity": (cpu or {}).get("parity"),
        "workloads": {k: {kk: (round(vv, 5) if isinstance(vv, float) else vv)
                          for kk, vv in v.items() if kk != "touched_experts_per_layer"}
                      for k, v in extras.items()},
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()

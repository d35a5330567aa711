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
EXPERT_BYTES_FULL = 14_450_688
METRIC = "MoE-layer tokens/s + achieved HBM GB/s (2-bit experts), decode and prefill"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=48)
    ap.add_argument("--workload", default="decode1")
    ap.add_argument("--extra", default="decode32_zipf,prefill2048,stack40_t64_zipf",
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


def traffic_record(kernel):
    """HBM traffic per launch from committed rocprofv3 counter runs, valid only while
    the kernel source is unchanged (sha256 recorded with the counters)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(kernel)
    if not rec:
        return None
    src = os.path.join(ROOT, rec["source"])
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if sha != rec["source_sha256"]:
        return None
    return rec


def run_workload(name, steps, warmup, rotate, graph=True):
    import torch
    import bit_quantized_routed_amd as mq
    from bit_quantized_routed_amd import workload as dw
    from synth import workloads as W

    wl = W.WORKLOADS[name]
    L = wl.layers if wl.layers > 1 else rotate
    t0 = time.time()
    tmp = torch.empty(wl.hidden * wl.inter, dtype=torch.float32, device="cuda")
    layers = [dw.DeviceLayer(wl, layer=l, tmp=tmp) for l in range(L)]
    del tmp
    torch.cuda.synchronize()
    log("[bench] %s: %d layer(s) generated in %.1fs" % (name, L, time.time() - t0))
    T, K, E = wl.tokens, wl.topk, wl.n_experts
    flags = mq.RESIDUAL_ADD if wl.rmsnorm else 0
    shape = layers[0].shape(flags)
    ws = dw.workspace(shape, T, K)
    x = dw.activations(wl)
    out = x if wl.rmsnorm else torch.empty((T, wl.hidden), dtype=torch.float32, device="cuda")
    counts = [torch.zeros(E, dtype=torch.int32, device="cuda") for _ in range(L)]
    stack = wl.layers > 1            # one step = the whole residual stack

    def one_pass(i, events=None):
        l = i % L
        tr = {"counts": counts[l]}
        if events is not None:
            tr["events"] = events
        mq.forward(x, layers[l].router_w, layers[l].experts, layers[l].shared_w, K, out, shape, T,
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
        # G consecutive steps per captured graph (one pass over the rotated layers
        # when that divides the step count, else one step), replayed steps / G times:
        # exactly `steps` steps, with one host launch per G steps
        G = L if (not stack and steps % L == 0) else 1
        n_graphs = 1 if (stack or G == L) else L
        graphs = []
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            for i in range(max(G, n_graphs)):
                step(i)
        torch.cuda.current_stream().wait_stream(cap)
        torch.cuda.synchronize()
        for j in range(n_graphs):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(G):
                    step(j + i)
            graphs.append(g)
        n_rep = steps // G
        for r in range(max(1, warmup // G)):
            graphs[r % n_graphs].replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for r in range(n_rep):
            graphs[r % n_graphs].replay()
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        ms_per_step = (t2 - t1) * 1e3 / (n_rep * G)
        launch = "hip_graph x%d steps" % G
        # spread of the step time: a separate pass of event-bracketed replays
        n_pct = max(10, min(60, n_rep))
        pev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n_pct)]
        for r in range(n_pct):
            pev[r][0].record()
            graphs[r % n_graphs].replay()
            pev[r][1].record()
        torch.cuda.synchronize()
        per_step = [a.elapsed_time(b) / G for a, b in pev]
        pct = {"p10": float(np.percentile(per_step, 10)), "p50": float(np.percentile(per_step, 50)),
               "p90": float(np.percentile(per_step, 90)), "replays": n_pct}
        del graphs
    touched = [int((c > 0).sum().item()) for c in counts]
    d_mean = float(np.mean(touched))
    passes = L if stack else 1
    tokens_per_step = T * (1 if not stack else 1)
    bytes_per_pass = layer_bytes(wl, d_mean)
    res = {
        "workload": name, "tokens": T, "layers_in_step": passes, "layers_resident": L,
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
    gu_bytes = d_mean * 2 * (wl.expert_bytes // 3)
    dn_bytes = d_mean * (wl.expert_bytes // 3)
    if T < 256 and wl.shared_inter and (wl.act == "bf16" or wl.rmsnorm):
        gu_bytes += 2 * wl.shared_inter * wl.hidden * 2
        dn_bytes += wl.shared_inter * wl.hidden * 2
    kbytes = {"gate_up": gu_bytes + T * wl.hidden * 2.5 + T * K * wl.inter * 4,
              "down": dn_bytes + T * K * wl.inter * 2.5 + T * K * wl.hidden * 4,
              "shared": 3 * wl.shared_inter * wl.hidden * 2}.get(dom)
    prefill = T >= 256
    if prefill:
        # useful MACs x 2 against the dense bf16 MFMA peak (the integer path issues two
        # int8 MACs per useful MAC, i.e. the same fraction of the int8 peak)
        kflops = {"gate_up": T * K * 2 * wl.inter * wl.hidden * 2,
                  "down": T * K * wl.hidden * wl.inter * 2,
                  "shared": T * 3 * wl.shared_inter * wl.hidden * 2}[dom]
        ach = kflops / (dom_avg * 1e-3) / 1e12
        res["roofline"] = {"bound": "mfma", "kernel": dom, "achieved": round(ach, 1),
                           "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                           "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                           "algorithmic_flops_per_launch": kflops, "avg_launch_ms": dom_avg}
        res["useful_tflops"] = (T * K * 3 * wl.inter * wl.hidden * 2 +
                                T * 3 * wl.shared_inter * wl.hidden * 2) / (ms_per_step * 1e-3) / 1e12
    elif kbytes is not None and dom_avg > 0:
        ach = kbytes / (dom_avg * 1e-3) / 1e9
        tr = traffic_record("%s/%s" % (name, dom))
        res["roofline"] = {"bound": "hbm", "kernel": dom, "achieved": round(ach, 1),
                           "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                           "traffic": None if tr is None else tr.get("bytes_per_launch"),
                           "algorithmic_bytes_per_launch": kbytes,
                           "avg_launch_ms": dom_avg}
    del layers, ws
    torch.cuda.empty_cache()
    return res


def W_layers(name):
    from synth import workloads as W
    return W.WORKLOADS[name].layers


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


def cpu_baseline(name, min_seconds=10.0, max_tokens=8):
    """The oracle, untuned, on the host cores for a bounded sample of the workload:
    the layer for its first tokens, one at a time, until at least min_seconds of
    oracle time (or max_tokens tokens); each token's routed experts are encoded to
    Q2 bytes beforehand, untimed (input preparation)."""
    from oracle import moe
    from tests.oracle_inputs import HostLayer
    from synth import workloads as W
    try:
        from threadpoolctl import threadpool_info
        thr = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        thr = 1
    wl = W.WORKLOADS[name]
    hl = HostLayer(wl, 0)
    xh, _ = W.activations(wl, tokens=max_tokens)
    idx, _, _, _ = moe.route(xh, hl.router_w, hl.router_b, wl.topk)
    total, n = 0.0, 0
    while n < max_tokens and total < min_seconds:
        for e in idx[n]:
            hl.expert_bytes(int(e))          # untimed: input preparation
        t = time.perf_counter()
        moe.layer(xh[n:n + 1], hl.router_w, hl.router_b, hl.expert_bytes, hl.shared, wl.topk, wl.hidden,
                  wl.inter)
        total += time.perf_counter() - t
        n += 1
    return {"value": round(n / total, 4), "unit": "tokens/s", "cores": int(thr),
            "affinity_cpus": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": "first %d token(s) of layer 0 of %s, one layer call each (routing, "
                      "dequantisation of the token's %d experts, fp64 FFNs, shared expert, combine); "
                      "%.2f s of oracle time" % (n, name, wl.topk, total)}


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
    cpu = cpu_baseline(args.workload) if args.cpu_baseline else None
    from synth import workloads as W
    wl = W.WORKLOADS[args.workload]
    line = {
        "metric": METRIC, "value": round(head["tokens_per_s"], 2), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp32", "data": "synthetic",
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
        "workloads": {k: {kk: (round(vv, 5) if isinstance(vv, float) else vv)
                          for kk, vv in v.items() if kk != "touched_experts_per_layer"}
                      for k, v in extras.items()},
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()

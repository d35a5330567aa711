"""Per-work-group timeline of the matrix-core decode launches of one layer call.

    python -m bit_quantized_routed_amd.timeline WORKLOAD [--calls N] [--rotate L]

Loads the diagnostic library libmoe_q2_timeline.so (built by
bit_quantized_routed_amd.build.build(timeline=True); the same sources compiled with
-DMQ_WG_TIMELINE) in place of libmoe_q2.so, materialises L distinct layers of the
workload, runs warm-up calls cycling through them, then N measured calls, each on the
next layer (its weights not in the last-level cache) after clearing the timestamp
array.  For each call and each of the two routed launches (gate/up, down) it prints,
per work-group role (routed unit, shared-expert rows, past the last unit), the count
and the percentiles of the start time, duration and end time relative to the launch's
first start, the routed work-groups' prologue (entry to the first column), the last
end per XCC, and the gap between the two launches.  Times are microseconds from the
device's constant 100 MHz clock.
"""
import argparse
import ctypes
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SLOTS, MAX_WG = 8, 16384
ROLES = ((0, "routed"), (1, "shared"), (2, "no work"))


def _pct(v):
    return "%.2f/%.2f/%.2f" % (np.percentile(v, 50), np.percentile(v, 90), v.max())


def summarise(buf):
    """Text lines for one call's timestamp array [2][MAX_WG][SLOTS] (kind 1 gate/up, 0 down)."""
    out = []
    spans = {}
    for kind, name in ((1, "gate/up"), (0, "down")):
        rec = buf[kind][buf[kind][:, 0] != 0]
        if not len(rec):
            continue
        t0, t1, t2 = (rec[:, i].astype(np.int64) for i in range(3))
        role, xcc = rec[:, 4].astype(np.int64), (rec[:, 3] & 0xF).astype(np.int64)
        base = t0.min()
        st, en = (t0 - base) / 100.0, (t2 - base) / 100.0
        spans[kind] = (t0.min(), t2.max())
        out.append("  %s launch: %d work-groups, last end %.2f us" % (name, len(rec), en.max()))
        for r, rname in ROLES:
            m = role == r
            if not m.any():
                continue
            line = "    %-8s n=%5d  start p50/p90/max %s  duration %s  end %s" % (
                rname, m.sum(), _pct(st[m]), _pct(en[m] - st[m]), _pct(en[m]))
            if r == 0:
                line += "  prologue %s" % _pct((t1[m] - t0[m]) / 100.0)
            out.append(line)
        out.append("    last end per XCC: " + " ".join(
            "%.1f" % en[xcc == i].max() if (xcc == i).any() else "-" for i in range(8)))
    if 0 in spans and 1 in spans:
        out.append("  gate/up last end -> down first start %.2f us; gate/up first start -> down last end %.2f us" % (
            (spans[0][0] - spans[1][1]) / 100.0, (spans[0][1] - spans[1][0]) / 100.0))
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("workload")
    ap.add_argument("--calls", type=int, default=3)
    ap.add_argument("--rotate", type=int, default=8)
    args = ap.parse_args()
    sys.path.insert(0, ROOT)
    import bit_quantized_routed_amd as mq
    mq.LIB_PATH = os.path.join(HERE, "libmoe_q2_timeline.so")
    if not os.path.exists(mq.LIB_PATH):
        raise SystemExit("libmoe_q2_timeline.so is not built: bit_quantized_routed_amd.build.build(timeline=True)")
    import torch
    from bit_quantized_routed_amd import workload as dw
    from synth import workloads as W

    lib = mq.library()
    lib.moe_q2_timeline_read.restype = ctypes.c_int
    lib.moe_q2_timeline_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    lib.moe_q2_timeline_clear.restype = ctypes.c_int
    wl = W.WORKLOADS[args.workload]
    if wl.layers > 1 or wl.rmsnorm:
        raise SystemExit("one-layer workloads only")
    tmp = torch.empty(wl.hidden * wl.inter, dtype=torch.float32, device="cuda")
    layers = [dw.DeviceLayer(wl, layer=l, tmp=tmp) for l in range(args.rotate)]
    del tmp
    x = dw.activations(wl)
    T, K = wl.tokens, wl.topk
    shape = layers[0].shape(0)
    plan = mq.describe(shape, T, K)
    if plan["path"] != mq.PATH_DECODE or plan["routed_kernel"] != 0:
        raise SystemExit("the workload does not run the matrix-core decode kernels")
    ws = torch.empty(mq.workspace_size(shape, T, K), dtype=torch.uint8, device="cuda")
    out = torch.empty((T, wl.hidden), dtype=torch.float32, device="cuda")

    def call(i):
        ly = layers[i % len(layers)]
        mq.forward(x, ly.router_w, ly.experts, ly.shared_w, K, out, shape, T, router_b=ly.router_b, workspace=ws)

    for i in range(3 * len(layers)):
        call(i)
    torch.cuda.synchronize()
    print("timeline of %s (T=%d, E=%d, K=%d, H=%d, I=%d; %d layers cycled; splits gate/up %d, down %d)" % (
        args.workload, T, wl.n_experts, K, wl.hidden, wl.inter, len(layers), plan["split_gate_up"],
        plan["split_down"]))
    buf = np.zeros((2, MAX_WG, SLOTS), dtype=np.uint64)
    for c in range(args.calls):
        assert lib.moe_q2_timeline_clear() == 0
        torch.cuda.synchronize()
        call(c)
        torch.cuda.synchronize()
        assert lib.moe_q2_timeline_read(buf.ctypes.data_as(ctypes.c_void_p), buf.nbytes) == 0
        print("call %d:" % c)
        print("\n".join(summarise(buf)), flush=True)


if __name__ == "__main__":
    main()

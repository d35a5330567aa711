"""GPU parity of the prefill workload (2048 tokens) and of the residual stack
(RMSNorm -> layer -> residual add) against the oracle."""
import numpy as np
import pytest
import torch

from oracle import moe
from synth import workloads as W
from tests.gpu_util import need_gpu, make_trace, trace_np, check_routing, rel_err, NEAR_TIE
from tests.oracle_inputs import HostLayer

pytestmark = pytest.mark.gpu

# The routed kernels of both paths (decode and prefill) multiply exact integer codes
# by two-digit (15-bit) activations and fold each block in fp32, so the prefill path
# is held to the same 2e-3 as the fp32-accumulate class (its observed error is ~3e-4).
TOL = 2e-3
# Free-running multi-layer comparison: after the first layer the two sides' residual
# streams differ at the 1e-4 level, and bf16 rounding of the RMSNorm output turns
# that into logit differences of up to ~1e-3; tokens whose oracle margin falls below
# DRIFT_TIE at a later layer are excluded (counted) from the output comparison.
DRIFT_TIE = 3e-3


def _bucket_property(tr, E, K):
    idx = tr["topk_idx"].reshape(-1)
    counts = np.bincount(idx, minlength=E)
    assert np.array_equal(tr["counts"], counts)
    assert np.array_equal(tr["offsets"], np.concatenate([[0], np.cumsum(counts)]))
    assert np.array_equal(tr["perm"], np.argsort(idx, kind="stable"))


@pytest.mark.parametrize("name,unit,act", [("prefill2048", 80, "exact"), ("prefill2048_q4", 64, "exact"),
                                            ("prefill2048", 80, "q8"), ("prefill2048_q4", 80, "q8")],
                         ids=["q2", "q4", "q2_act_q8", "q4_act_q8"])
def test_prefill2048_sampled(name, unit, act):
    """64 tokens of the 2048-token prefill (2-bit layer: 80-slot work units; 4-bit
    layer: 64-slot units with two-digit activations, 80 with Q8 activations, which are
    checked against the oracle's Q8 mode): for every bucket larger than one work unit,
    the token of its last slot and of the first slot of its second unit, tokens 0 and
    2047, the rest seeded at random."""
    mq = need_gpu()
    from bit_quantized_routed_amd import workload as dw
    from tests.oracle_pool import ExpertPool, layer_outputs
    wl = W.WORKLOADS[name]
    dl = dw.DeviceLayer(wl)
    T, K = wl.tokens, wl.topk
    shape = dl.shape(mq.ACT_Q8 if act == "q8" else 0)
    assert mq.describe(shape, T, K)["routed_kernel"] == 2
    ws = dw.workspace(shape, T, K)
    tr = make_trace(T, K, wl.n_experts)
    out = torch.zeros((T, wl.hidden), dtype=torch.float32, device="cuda")
    x = dw.activations(wl)
    mq.forward(x, dl.router_w, dl.experts, dl.shared_w, K, out, shape, T,
               router_b=dl.router_b, workspace=ws, trace=tr)
    torch.cuda.synchronize()
    print("  [prefill] GPU layer done", flush=True)
    o = out.cpu().numpy().astype(np.float64)
    trn = trace_np(tr)
    hl = HostLayer(wl)
    xh, _ = W.activations(wl)
    idx, g, logits, margin = moe.route(xh, hl.router_w, hl.router_b, K)
    route = {"idx": idx, "g": g, "logits": logits, "margin": margin}
    excluded, rep = check_routing(trn, route, wl.n_experts, K)
    print("  [prefill] routing and bucketing checked", rep, flush=True)
    off, perm = trn["offsets"], trn["perm"]
    big = np.nonzero(trn["counts"] > unit)[0]
    want = {0, T - 1}
    for e in big:
        want.add(int(perm[off[e + 1] - 1]) // K)
        want.add(int(perm[off[e] + unit]) // K)
    rng = np.random.default_rng(3)
    for t in rng.permutation(T):
        if len(want) >= 64:
            break
        want.add(int(t))
    sample = np.array(sorted(want))
    sample = sample[~excluded[sample]]
    pool = ExpertPool()
    try:
        (ref, _), = layer_outputs(pool, wl.name, [(0, hl, xh[sample])], K, wl.hidden, wl.inter, act=act)
    finally:
        pool.close()
    err = rel_err(o[sample], ref)
    print(name, act, rep, "tokens compared", sample.size, "buckets > %d slots" % unit, big.size,
          "rel_err", err, "bucket sizes min/max", int(trn["counts"].min()), int(trn["counts"].max()))
    assert sample.size >= 60
    assert err <= TOL


def _run_stack(mq, dw, wl, n_layers, tokens=None):
    """GPU residual stack over the first n_layers layers; returns the final stream and
    the per-layer traces."""
    T = wl.tokens if tokens is None else tokens
    h = dw.activations(wl, tokens=T)
    traces = []
    for l in range(n_layers):
        dl = dw.DeviceLayer(wl, layer=l)
        shape = dl.shape(mq.RESIDUAL_ADD)
        ws = dw.workspace(shape, T, wl.topk)
        tr = make_trace(T, wl.topk, wl.n_experts)
        mq.forward(h, dl.router_w, dl.experts, dl.shared_w, wl.topk, h, shape, T,
                   router_b=dl.router_b, workspace=ws, trace=tr)
        torch.cuda.synchronize()
        print("  [stack] GPU layer %d done" % l, flush=True)
        traces.append(trace_np(tr))
        del dl, ws
    return h.cpu().numpy().astype(np.float64), traces


def _compare_stack(wl, h_gpu, traces, ref_h, routings, toks):
    """Routing per layer (sets), bucketing property per layer, final stream."""
    K, E = wl.topk, wl.n_experts
    keep = np.ones(len(toks), dtype=bool)
    for l, (tr, r) in enumerate(zip(traces, routings)):
        _bucket_property(tr, E, K)
        tie = NEAR_TIE if l == 0 else DRIFT_TIE
        for i, t in enumerate(toks):
            if r["margin"][i] < tie:
                keep[i] = False
            if keep[i]:
                assert set(tr["topk_idx"][t].tolist()) == set(r["idx"][i].tolist()), (l, t)
    err = rel_err(h_gpu[toks][keep], ref_h[keep]) if keep.any() else 0.0
    return err, int((~keep).sum())


def test_tiny_stack_all_tokens():
    mq = need_gpu()
    from bit_quantized_routed_amd import workload as dw
    wl = W.WORKLOADS["tiny_stack"]
    h_gpu, traces = _run_stack(mq, dw, wl, wl.layers)
    layers = [HostLayer(wl, l).oracle_layer() for l in range(wl.layers)]
    h0, _ = W.activations(wl)
    ref, routings = moe.stack(h0, layers, wl.topk, wl.hidden, wl.inter, wl.rms_eps)
    toks = np.arange(wl.tokens)
    err, excl = _compare_stack(wl, h_gpu, traces, ref, routings, toks)
    print("tiny_stack layers", wl.layers, "excluded", excl, "rel_err", err)
    assert excl < wl.tokens // 2
    assert err <= TOL


def _shared_sample(idx, excluded, first, n):
    """`first` (or the last token before it that is not a near tie) and n - 1 more
    tokens, each chosen to add the fewest experts not yet in the sample's union (ties:
    lower token), so the oracle evaluates few distinct experts."""
    T = idx.shape[0]
    t0 = first
    while excluded[t0]:
        t0 -= 1
    toks, union = [t0], set(idx[t0].tolist())
    while len(toks) < n:
        best = min((len(set(idx[t].tolist()) - union), t) for t in range(T) if t not in toks and not excluded[t])
        toks.append(best[1])
        union |= set(idx[best[1]].tolist())
    return sorted(toks)


def test_stack40_every_layer():
    """Each of the 40 layers of the deep stack on its own residual input h_l (a seeded
    fp32 draw of the layer's stream, identical on both sides; no value goes from the
    GPU into the oracle): RMSNorm -> layer -> residual add in place on the device;
    routing of all 64 tokens and the bucketing checked per layer, and the layer's
    increment out - h_l of 4 tokens (token 63 among them) compared with the oracle's
    layer output on bf16(RMSNorm(h_l))."""
    mq = need_gpu()
    from bit_quantized_routed_amd import workload as dw
    from tests.oracle_pool import ExpertPool, layer_outputs
    wl = W.WORKLOADS["stack40_t64_zipf"]
    T, K, E = wl.tokens, wl.topk, wl.n_experts
    jobs, gpu_inc, n_excl = [], [], 0
    tmp = torch.empty(wl.hidden * wl.inter, dtype=torch.float32, device="cuda")
    for l in range(wl.layers):
        dl = dw.DeviceLayer(wl, layer=l, tmp=tmp)
        h = dw.layer_residual(wl, l)
        h_in = h.clone()
        shape = dl.shape(mq.RESIDUAL_ADD)
        ws = dw.workspace(shape, T, K)
        tr = make_trace(T, K, E)
        mq.forward(h, dl.router_w, dl.experts, dl.shared_w, K, h, shape, T,
                   router_b=dl.router_b, workspace=ws, trace=tr)
        torch.cuda.synchronize()
        inc = (h.cpu().numpy().astype(np.float64) - h_in.cpu().numpy().astype(np.float64))
        trn = trace_np(tr)
        del dl, ws, h, h_in
        hh = W.layer_residual(wl, l)
        hl = HostLayer(wl, l)
        xl = moe.rmsnorm_bf16(hh, wl.rms_eps)
        idx, g, logits, margin = moe.route(xl, hl.router_w, hl.router_b, K)
        excluded, rep = check_routing(trn, {"idx": idx, "g": g, "logits": logits, "margin": margin}, E, K)
        n_excl += int(excluded.sum())
        toks = _shared_sample(idx, excluded, T - 1, 4)
        jobs.append((l, hl, xl[toks]))
        gpu_inc.append(inc[toks])
        print("  [stack40] layer %d: GPU done, routing checked %s, tokens %s" % (l, rep, toks), flush=True)
    del tmp
    torch.cuda.empty_cache()
    pool = ExpertPool()
    try:
        refs = layer_outputs(pool, wl.name, jobs, K, wl.hidden, wl.inter)
    finally:
        pool.close()
    errs = [rel_err(inc, ref) for inc, (ref, _) in zip(gpu_inc, refs)]
    print("stack40 per layer: near-tie tokens", n_excl, "max rel_err", max(errs),
          "per layer", ["%.2e" % e for e in errs])
    assert max(errs) <= TOL


# Bound of the chained drift report: each layer's own error is ~2e-4 (the per-layer
# test), but a 1e-4 difference of the residual streams moves some RMSNorm outputs
# across a bf16 rounding boundary (one bf16 ulp, 2^-8 relative, of that element of the
# next layer's input), which the next layers carry on; 3 chained layers measured 1.9e-3.
DRIFT_TOL = 5e-3


def test_stack40_first_layers_chained():
    """Drift report: the first 3 layers chained free-running from h_0 on both sides
    (the per-layer check above is the parity test); at least 2 of the 4 tokens stay
    outside the widening near-tie window and are compared, within DRIFT_TOL."""
    mq = need_gpu()
    from bit_quantized_routed_amd import workload as dw
    from tests.oracle_pool import ExpertPool
    wl = W.WORKLOADS["stack40_t64_zipf"]
    n_layers = 3
    h_gpu, traces = _run_stack(mq, dw, wl, n_layers)
    toks = np.array([5, 22, 40, 63])
    pool = ExpertPool()
    try:
        layers = []
        for l in range(n_layers):
            L = HostLayer(wl, l).oracle_layer()
            L["ffn_map"] = pool.ffn_map(wl.name, l)
            layers.append(L)
        h0, _ = W.activations(wl)
        ref, routings = moe.stack(h0[toks], layers, wl.topk, wl.hidden, wl.inter, wl.rms_eps)
    finally:
        pool.close()
    # all 64 tokens' first-layer routing (identical inputs on both sides)
    hl0 = HostLayer(wl, 0)
    idx, g, logits, margin = moe.route(moe.rmsnorm_bf16(h0, wl.rms_eps), hl0.router_w, hl0.router_b,
                                       wl.topk)
    check_routing(traces[0], {"idx": idx, "g": g, "logits": logits, "margin": margin},
                  wl.n_experts, wl.topk)
    err, excl = _compare_stack(wl, h_gpu, traces, ref, routings, toks)
    print("stack40 first", n_layers, "layers chained, tokens", toks.tolist(), "excluded", excl, "rel_err", err)
    assert len(toks) - excl >= 2
    assert err <= DRIFT_TOL

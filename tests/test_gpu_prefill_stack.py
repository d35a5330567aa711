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

TOL_PREFILL = 1e-2
TOL_DECODE = 2e-3
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


def test_prefill2048_sampled():
    mq = need_gpu()
    from bit_quantized_routed_amd import workload as dw
    from tests.oracle_pool import ExpertPool
    wl = W.WORKLOADS["prefill2048"]
    dl = dw.DeviceLayer(wl)
    T = wl.tokens
    shape = dl.shape()
    ws = dw.workspace(shape, T, wl.topk)
    tr = make_trace(T, wl.topk, wl.n_experts)
    out = torch.zeros((T, wl.hidden), dtype=torch.float32, device="cuda")
    x = dw.activations(wl)
    mq.forward(x, dl.router_w, dl.experts, dl.shared_w, wl.topk, out, shape, T,
               router_b=dl.router_b, workspace=ws, trace=tr)
    torch.cuda.synchronize()
    print("  [prefill] GPU layer done", flush=True)
    o = out.cpu().numpy().astype(np.float64)
    trn = trace_np(tr)
    hl = HostLayer(wl)
    xh, _ = W.activations(wl)
    idx, g, logits, margin = moe.route(xh, hl.router_w, hl.router_b, wl.topk)
    route = {"idx": idx, "g": g, "logits": logits, "margin": margin}
    excluded, rep = check_routing(trn, route, wl.n_experts, wl.topk)
    print("  [prefill] routing and bucketing checked", rep, flush=True)
    sample = np.array([0, 777, 2047])
    sample = sample[~excluded[sample]]
    pool = ExpertPool()
    try:
        ref, _ = moe.layer(xh[sample], hl.router_w, hl.router_b, None, hl.shared, wl.topk,
                           wl.hidden, wl.inter, ffn_map=pool.ffn_map(wl.name, 0))
    finally:
        pool.close()
    err = rel_err(o[sample], ref)
    print("prefill2048", rep, "tokens", sample.tolist(), "rel_err", err,
          "bucket sizes min/max", int(trn["counts"].min()), int(trn["counts"].max()))
    assert err <= TOL_PREFILL


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
    assert err <= TOL_DECODE


def test_stack40_first_layers_sampled():
    mq = need_gpu()
    from bit_quantized_routed_amd import workload as dw
    from tests.oracle_pool import ExpertPool
    wl = W.WORKLOADS["stack40_t64_zipf"]
    n_layers = 3
    h_gpu, traces = _run_stack(mq, dw, wl, n_layers)
    toks = np.array([5, 40])
    pool = ExpertPool()
    try:
        layers = []
        for l in range(n_layers):
            hl = HostLayer(wl, l)
            L = hl.oracle_layer()
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
    print("stack40 first", n_layers, "layers, tokens", toks.tolist(), "excluded", excl, "rel_err", err)
    assert err <= TOL_DECODE

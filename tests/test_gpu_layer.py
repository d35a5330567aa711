"""GPU parity of the whole layer against the oracle (HIP path through the C ABI)."""
import functools

import numpy as np
import pytest
import torch

from oracle import moe
from synth import workloads as W
from tests.gpu_util import need_gpu, make_trace, trace_np, check_routing, rel_err
from tests.oracle_inputs import host_layer

pytestmark = pytest.mark.gpu

TOL_DECODE = 2e-3


def _run(mq, dl, x, T, flags=0, out=None):
    from bit_quantized_routed_amd import workload as dw
    wl = dl.wl
    shape = dl.shape(flags)
    ws = dw.workspace(shape, T, wl.topk)
    tr = make_trace(T, wl.topk, wl.n_experts)
    if out is None:
        out = torch.zeros((T, wl.hidden), dtype=torch.float32, device="cuda")
    mq.forward(x, dl.router_w, dl.experts, dl.shared_w, wl.topk, out, shape, T,
               router_b=dl.router_b, workspace=ws, trace=tr)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), trace_np(tr)


@pytest.mark.parametrize("kernel", ["mma", "valu"])
def test_tiny_layer(kernel):
    mq = need_gpu()
    from bit_quantized_routed_amd import workload as dw
    wl = W.WORKLOADS["tiny"]
    dl = dw.DeviceLayer(wl)
    hl = host_layer("tiny")
    assert np.array_equal(dl.experts.cpu().numpy(), hl.all_expert_bytes())
    x = dw.activations(wl)
    out, tr = _run(mq, dl, x, wl.tokens, flags=mq.DECODE_VALU if kernel == "valu" else 0)
    xh, _ = W.activations(wl)
    assert np.array_equal(x.cpu().numpy(), xh)
    ref, route = moe.layer(xh, hl.router_w, hl.router_b, hl.expert_bytes, hl.shared, wl.topk,
                           wl.hidden, wl.inter)
    excluded, rep = check_routing(tr, route, wl.n_experts, wl.topk)
    err = rel_err(out, ref, ~excluded)
    print("tiny", rep, "rel_err", err)
    assert err <= TOL_DECODE


@functools.lru_cache(maxsize=4)
def _pooled_ref(name, toks):
    """Oracle outputs of the given tokens of layer 0 (experts evaluated in parallel;
    cached, several tests compare different kernels against the same tokens)."""
    from tests.oracle_pool import ExpertPool, layer_outputs
    wl = W.WORKLOADS[name]
    xh, _ = W.activations(wl)
    pool = ExpertPool()
    try:
        (ref, _), = layer_outputs(pool, name, [(0, host_layer(name), xh[list(toks)])], wl.topk, wl.hidden,
                                  wl.inter)
    finally:
        pool.close()
    return ref


def _full_check(name, sample=None, flags=0, pooled=False):
    """The layer at full size: every token's routing and the bucketing, and the
    outputs of the sampled tokens (all by default) against the oracle."""
    mq = need_gpu()
    from bit_quantized_routed_amd import workload as dw
    wl = W.WORKLOADS[name]
    dl = dw.DeviceLayer(wl)
    hl = host_layer(name)
    x = dw.activations(wl)
    out, tr = _run(mq, dl, x, wl.tokens, flags=flags)
    xh, _ = W.activations(wl)
    # routing for every token (router only), bucketing exactly
    idx, g, logits, margin = moe.route(xh, hl.router_w, hl.router_b, wl.topk)
    route = {"idx": idx, "g": g, "logits": logits, "margin": margin}
    excluded, rep = check_routing(tr, route, wl.n_experts, wl.topk)
    toks = np.arange(wl.tokens) if sample is None else np.asarray(sample)
    toks = toks[~excluded[toks]]
    if pooled:
        ref = _pooled_ref(name, tuple(int(t) for t in toks))
    else:
        ref, _ = moe.layer(xh[toks], hl.router_w, hl.router_b, hl.expert_bytes, hl.shared, wl.topk,
                           wl.hidden, wl.inter)
    err = rel_err(out[toks], ref)
    print(name, rep, "tokens compared", toks.size, "rel_err", err)
    assert toks.size >= (wl.tokens if sample is None else len(sample)) - 2
    assert err <= TOL_DECODE
    return err


@pytest.mark.parametrize("kernel", ["mma", "valu", "mma_serial"])
def test_decode1_layer(kernel):
    import bit_quantized_routed_amd as mq
    flags = {"mma": 0, "valu": mq.DECODE_VALU, "mma_serial": mq.SERIAL}[kernel]
    _full_check("decode1", flags=flags)


# (workload, flags) pairs whose activation preparation and shared expert run on the
# internal concurrent stream: the prefill kernels with a shared expert, the vector-ALU
# decode kernel, an fp32 layer input
SIDE_BRANCH = [("decode32_zipf", "PATH_PREFILL"), ("decode32_zipf", "DECODE_VALU"), ("tiny", "")]


@pytest.mark.parametrize("name,flag", SIDE_BRANCH)
def test_shared_branch_concurrent_equals_serial(name, flag):
    """The concurrent branch forked onto the internal stream gives the same bits as
    the all-on-one-stream order, over several back-to-back calls (the plan confirms
    that the branch is in use, so the comparison is not between two identical paths)."""
    mq = need_gpu()
    from bit_quantized_routed_amd import workload as dw
    wl = W.WORKLOADS[name]
    f = getattr(mq, flag) if flag else 0
    dl = dw.DeviceLayer(wl)
    plan = mq.describe(dl.shape(f), wl.tokens, wl.topk)
    assert plan["side_branch"] == 1 and plan["shared_fused"] == 0, plan
    assert mq.describe(dl.shape(f | mq.SERIAL), wl.tokens, wl.topk)["side_branch"] == 0
    x = dw.activations(wl)
    ser, _ = _run(mq, dl, x, wl.tokens, flags=f | mq.SERIAL)
    for _ in range(3):
        con, _ = _run(mq, dl, x, wl.tokens, flags=f)
        assert np.array_equal(con, ser)


@pytest.mark.parametrize("kernel", ["mma", "valu"])
def test_decode32_zipf_layer_all_tokens(kernel):
    import bit_quantized_routed_amd as mq
    _full_check("decode32_zipf", flags=mq.DECODE_VALU if kernel == "valu" else 0, pooled=True)


@pytest.mark.parametrize("T", [2, 3, 4, 5, 8, 9])
def test_small_batches(T):
    """Small batches of the decode shape: up to 4 tokens the top-K and the bucketing
    run as one work-group, from 5 on as two launches; up to 8 tokens the router
    runs one work-group per expert, from 9 on on the matrix cores with split-K.
    Routing and bucketing of every token, the output of the last."""
    mq = need_gpu()
    from bit_quantized_routed_amd import workload as dw
    wl = W.WORKLOADS["decode32_zipf"]
    dl = dw.DeviceLayer(wl)
    hl = host_layer("decode32_zipf")
    x = dw.activations(wl, tokens=T)
    out, tr = _run(mq, dl, x, T)
    xh, _ = W.activations(wl, tokens=T)
    idx, g, logits, margin = moe.route(xh, hl.router_w, hl.router_b, wl.topk)
    excluded, rep = check_routing(tr, {"idx": idx, "g": g, "logits": logits, "margin": margin},
                                  wl.n_experts, wl.topk)
    assert not excluded[T - 1]
    ref, _ = moe.layer(xh[T - 1:T], hl.router_w, hl.router_b, hl.expert_bytes, hl.shared, wl.topk,
                       wl.hidden, wl.inter)
    err = rel_err(out[T - 1:T], ref)
    print("decode32_zipf first", T, rep, "rel_err", err)
    assert err <= TOL_DECODE


def test_decode32_forced_prefill_kernels():
    """The prefill kernels on a decode-sized batch (PATH_PREFILL), all 32 tokens through
    the oracle: covers partial token fragments and buckets of 1..18 slots."""
    import bit_quantized_routed_amd as mq
    _full_check("decode32_zipf", flags=mq.PATH_PREFILL, pooled=True)


def test_tiny_forced_prefill_kernels():
    """Prefill kernels at the tiny shape: 1-block reduction rows (H = 256) and a
    2-block down projection, fewer rows than one 256-row super-tile."""
    import bit_quantized_routed_amd as mq
    _full_check("tiny", flags=mq.PATH_PREFILL)

"""Combinations of the layer's options on the GPU.

Batch invariance with Q8 activations and with the 4-bit format, at a shape (hidden
2048, intermediate 2048, 64 experts, top-8; the mid_e64 workloads) where a token alone runs the fixed
reduction splits as separate work-groups and a 24-token batch runs them merged:
the token's outputs, routing and gates are the same bits alone, in a 3-token and in
the 24-token batch, and the batch agrees with the oracle (Q8 mode for Q8).  The
expert cache with those options gives the resident layer's bits."""
import numpy as np
import pytest
import torch

from oracle import moe
from synth import workloads as W
from tests.gpu_util import need_gpu, make_trace, trace_np, check_routing, rel_err
from tests.oracle_inputs import HostLayer

pytestmark = pytest.mark.gpu

TOL = 2e-3

# workload, flag names
CASES = [
    ("mid_e64", ("BATCH_INVARIANT", "ACT_Q8")),
    ("mid_e64_q4", ("BATCH_INVARIANT",)),
    ("mid_e64_q4gu", ("BATCH_INVARIANT", "ACT_Q8")),
]


@pytest.fixture(scope="module")
def pool():
    from tests.oracle_pool import ExpertPool
    p = ExpertPool()
    yield p
    p.close()


def _flags(mq, names):
    f = 0
    for n in names:
        f |= getattr(mq, n)
    return f


def _run(mq, dl, x, T, flags):
    from bit_quantized_routed_amd import workload as dw
    wl = dl.wl
    shape = dl.shape(flags)
    ws = dw.workspace(shape, T, wl.topk)
    tr = make_trace(T, wl.topk, wl.n_experts)
    out = torch.zeros((T, wl.hidden), dtype=torch.float32, device="cuda")
    mq.forward(x, dl.router_w, dl.experts, dl.shared_w, wl.topk, out, shape, T, router_b=dl.router_b,
               workspace=ws, trace=tr)
    torch.cuda.synchronize()
    return out.cpu().numpy(), trace_np(tr)


@pytest.mark.parametrize("case", CASES, ids=["_".join((c[0],) + c[1]) for c in CASES])
def test_batch_invariance_with_formats(case, pool):
    mq = need_gpu()
    from bit_quantized_routed_amd import workload as dw
    from tests.oracle_pool import layer_outputs
    name, names = case
    wl = W.WORKLOADS[name]
    T, H, E, K, I = wl.tokens, wl.hidden, wl.n_experts, wl.topk, wl.inter
    dl = dw.DeviceLayer(wl)
    flags = _flags(mq, names)
    shape = dl.shape(flags)
    one, batch = mq.describe(shape, 1, K), mq.describe(shape, T, K)
    assert one["merged"] == 0 and batch["merged"] == 1 and one["split_gate_up"] > 1
    assert (one["split_gate_up"], one["split_down"]) == (batch["split_gate_up"], batch["split_down"])
    x = dw.activations(wl)
    out, tr = _run(mq, dl, x, T, flags)
    for t in (0, 7, T - 1):
        for lo, n in ((t, 1), (3 * (t // 3), 3)):
            o, trs = _run(mq, dl, x[lo:lo + n].contiguous(), n, flags)
            assert np.array_equal(o[t - lo], out[t]), (name, t, n)
            assert np.array_equal(trs["topk_idx"][t - lo], tr["topk_idx"][t])
            assert np.array_equal(trs["topk_w"][t - lo], tr["topk_w"][t])
    # the batch against the oracle (Q8 mode under ACT_Q8)
    hl = HostLayer(wl)
    xh, _ = W.activations(wl)
    idx, g, logits, margin = moe.route(xh, hl.router_w, hl.router_b, K)
    excluded, rep = check_routing(tr, {"idx": idx, "g": g, "logits": logits, "margin": margin}, E, K)
    toks = np.arange(T)[~excluded]
    assert toks.size >= T - 2
    a = "q8" if "ACT_Q8" in names else "exact"
    (ref, _), = layer_outputs(pool, name, [(0, hl, xh[toks])], K, H, I, act=a)
    err = rel_err(out[toks].astype(np.float64), ref)
    print(name, names, rep, "tokens compared", toks.size, "rel_err", err, flush=True)
    assert err <= TOL


@pytest.mark.parametrize("names", [("ACT_Q8",), ("BATCH_INVARIANT",), ("BATCH_INVARIANT", "ACT_Q8")],
                         ids=["q8", "bi", "bi_q8"])
def test_cache_with_options(names):
    """moe_q2_forward_cached under Q8 / batch-invariant flags, a 16-slot budget for
    calls touching up to ~60 of 64 experts (misses cached and uncached): the resident
    layer's bits with the same flags."""
    mq = need_gpu()
    from bit_quantized_routed_amd import workload as dw
    wl = W.WORKLOADS["mid_e64_q4dn"]
    dl = dw.DeviceLayer(wl)
    flags = _flags(mq, names)
    shape = dl.shape(flags)
    T, K, E = wl.tokens, wl.topk, wl.n_experts
    host = torch.empty(dl.experts.numel(), dtype=torch.uint8, pin_memory=True)
    host.copy_(dl.experts)
    torch.cuda.synchronize()
    slots = torch.empty(16 * wl.expert_bytes, dtype=torch.uint8, device="cuda")
    state = torch.empty(mq.cache_state_bytes(16, E) // 4, dtype=torch.int32, device="cuda")
    cache = mq.make_cache(slots, wl.expert_bytes, 16, E, state)
    mq.cache_reset(cache)
    ws = dw.workspace(shape, T, K)
    xs = dw.activations(wl, tokens=3 * T)
    for b in (0, 1, 0, 2):
        x = xs[b * T:(b + 1) * T].contiguous()
        ref, _ = _run(mq, dl, x, T, flags)
        out = torch.full((T, wl.hidden), 7.0, dtype=torch.float32, device="cuda")
        mq.forward_cached(x, dl.router_w, host, 0, cache, dl.shared_w, K, out, shape, T, router_b=dl.router_b,
                          workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), ref), (names, b)

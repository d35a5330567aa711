"""moe_q2_forward_noalloc, the entry point for callers that cannot allocate, against
moe_q2_forward on the same inputs through the C ABI: identical outputs and routing
on two calls in a row, the second with a smaller batch (the fixed per-device
workspace keeps the first call's contents), on the fused decode path, on a path
whose normal entry point forks the internal stream (an fp32 layer input), and on the
residual stack updated in place."""
import numpy as np
import pytest
import torch

from synth import workloads as W
from tests.gpu_util import need_gpu, make_trace, trace_np

pytestmark = pytest.mark.gpu


def _both(mq, dw, dl, wl, T, flags=0, in_place=False):
    shape = dl.shape(flags)
    K = wl.topk
    x = dw.layer_residual(wl, 0, tokens=T) if in_place else dw.activations(wl, tokens=T)
    res = []
    for entry in ("forward", "noalloc"):
        xx = x.clone()
        out = xx if in_place else torch.full((T, wl.hidden), 3.0, dtype=torch.float32, device="cuda")
        tr = make_trace(T, K, wl.n_experts)
        if entry == "forward":
            ws = dw.workspace(shape, T, K)
            mq.forward(xx, dl.router_w, dl.experts, dl.shared_w, K, out, shape, T, router_b=dl.router_b,
                       workspace=ws, trace=tr)
        else:
            mq.forward_noalloc(xx, dl.router_w, dl.experts, dl.shared_w, K, out, shape, T,
                               router_b=dl.router_b, trace=tr)
        torch.cuda.synchronize()
        res.append((out.cpu().numpy(), trace_np(tr)))
    (o1, t1), (o2, t2) = res
    assert np.array_equal(o1, o2), (wl.name, T)
    for k in t1:
        assert np.array_equal(t1[k], t2[k]), (wl.name, T, k)
    return o1


@pytest.mark.parametrize("name,tokens", [("decode32_zipf", (32, 5)), ("tiny", (4, 2))])
def test_noalloc_equals_forward_twice(name, tokens):
    mq = need_gpu()
    from bit_quantized_routed_amd import workload as dw
    wl = W.WORKLOADS[name]
    dl = dw.DeviceLayer(wl)
    if name == "tiny":            # fp32 input: the workspace entry point forks its internal stream
        assert mq.describe(dl.shape(0), wl.tokens, wl.topk)["side_branch"] == 1
    for T in tokens:              # two calls in a row, the second smaller
        print("  [noalloc]", name, "T =", T, flush=True)
        _both(mq, dw, dl, wl, T)


def test_noalloc_residual_stack_in_place():
    mq = need_gpu()
    from bit_quantized_routed_amd import workload as dw
    wl = W.WORKLOADS["tiny_stack"]
    dl = dw.DeviceLayer(wl)
    for T in (16, 3):
        print("  [noalloc] tiny_stack in place, T =", T, flush=True)
        _both(mq, dw, dl, wl, T, flags=mq.RESIDUAL_ADD, in_place=True)


def test_noalloc_refuses_large_batch_before_enqueue():
    mq = need_gpu()
    wl = W.WORKLOADS["decode32_zipf"]
    shape = mq.make_shape(wl.hidden, wl.inter, wl.n_experts, wl.shared_inter, mq.BF16)
    T = 255                       # the decode path's workspace at 255 tokens: 207 MiB
    assert mq.workspace_size(shape, T, wl.topk) > mq.NOALLOC_MAX_BYTES
    x = torch.zeros((T, wl.hidden), dtype=torch.bfloat16, device="cuda")
    out = torch.full((T, wl.hidden), 5.0, dtype=torch.float32, device="cuda")
    wr = torch.zeros((wl.n_experts, wl.hidden), dtype=torch.float32, device="cuda")
    ex = torch.zeros(16, dtype=torch.uint8, device="cuda")       # never read: refused first
    sh = torch.zeros(16, dtype=torch.bfloat16, device="cuda")
    rc = mq.forward_noalloc(x, wr, ex, sh, wl.topk, out, shape, T, check=False)
    assert rc == mq.EUNSUPPORTED
    torch.cuda.synchronize()
    assert torch.all(out == 5.0)


def test_noalloc_with_options():
    """Batch-invariant 4-bit layer: a 24-token call (merged split work-groups) and then
    a one-token call (one work-group per split) on the fixed workspace."""
    mq = need_gpu()
    from bit_quantized_routed_amd import workload as dw
    wl = W.WORKLOADS["mid_e64_q4"]
    dl = dw.DeviceLayer(wl)
    for T in (24, 1):
        print("  [noalloc] mid_e64_q4 batch-invariant T =", T, flush=True)
        _both(mq, dw, dl, wl, T, flags=mq.BATCH_INVARIANT)

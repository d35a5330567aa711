"""HIP graph capture of moe_q2_forward (with its concurrent branch): every replay,
with eager calls and synchronisations in between, equals the eager result bit for
bit."""
import pytest
import torch

from synth import workloads as W
from tests.gpu_util import need_gpu

pytestmark = pytest.mark.gpu


# The fused decode path (one stream) and the paths whose concurrent branch is forked
# onto the internal stream inside the capture (prefill kernels with a shared expert,
# the vector-ALU decode kernel, an fp32 layer input).
GRAPH_CASES = [("decode1", ""), ("decode32_zipf", ""), ("tiny_stack", ""),
               ("decode32_zipf", "PATH_PREFILL"), ("decode32_zipf", "DECODE_VALU"), ("tiny", "")]


@pytest.mark.parametrize("name,flag", GRAPH_CASES)
def test_graph_replays_equal_eager(name, flag):
    mq = need_gpu()
    from bit_quantized_routed_amd import workload as dw
    wl = W.WORKLOADS[name]
    dl = dw.DeviceLayer(wl)
    T, K = wl.tokens, wl.topk
    shape = dl.shape(getattr(mq, flag) if flag else 0)      # PRE_RMSNORM for the stack shape
    plan = mq.describe(shape, T, K)
    assert plan["side_branch"] == (0 if plan["shared_fused"] else 1), plan
    if flag or name == "tiny":
        assert plan["side_branch"] == 1
    ws = dw.workspace(shape, T, K)
    x = dw.activations(wl)
    out_e = torch.empty((T, wl.hidden), dtype=torch.float32, device="cuda")
    out_g = torch.empty_like(out_e)

    def fwd(out):
        mq.forward(x, dl.router_w, dl.experts, dl.shared_w, K, out, shape, T,
                   router_b=dl.router_b, workspace=ws)

    fwd(out_e)
    torch.cuda.synchronize()
    ref = out_e.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fwd(out_g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fwd(out_g)
    for rep in range(4):
        out_g.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, ref), "replay %d differs from the eager result" % rep
        fwd(out_e)                       # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out_e, ref)


def test_graph_with_phase_events_and_kernel_timing():
    """Timing events passed in the trace: eagerly the routed-expert kernels record them
    on their own dispatch (a positive duration, the same output); under capture they are
    recorded around plain launches, and the replays still equal the eager result."""
    mq = need_gpu()
    from bit_quantized_routed_amd import workload as dw
    wl = W.WORKLOADS["decode1"]
    dl = dw.DeviceLayer(wl)
    T, K = wl.tokens, wl.topk
    shape = dl.shape(0)
    ws = dw.workspace(shape, T, K)
    x = dw.activations(wl)
    out_e = torch.empty((T, wl.hidden), dtype=torch.float32, device="cuda")
    out_g = torch.empty_like(out_e)
    ev = mq.EventSet()

    def fwd(out, events):
        tr = {"events": events} if events is not None else None
        mq.forward(x, dl.router_w, dl.experts, dl.shared_w, K, out, shape, T,
                   router_b=dl.router_b, workspace=ws, trace=tr)

    fwd(out_e, None)
    torch.cuda.synchronize()
    ref = out_e.clone()
    fwd(out_e, ev)
    el = ev.elapsed()
    assert torch.equal(out_e, ref)
    assert el["gate_up"] > 0 and el["down"] > 0, el
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fwd(out_g, ev)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fwd(out_g, ev)
    for rep in range(3):
        out_g.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, ref), "replay %d differs from the eager result" % rep
    ev.close()

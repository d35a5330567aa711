"""The C ABI from a plain C program (tests/c/moe_q2_consumer.c: HIP runtime from C,
its own hipMalloc'd buffers, no torch): the same layer inputs give the same output
and routing bits as the Python binding's call, and invalid arguments come back as
statuses.  The program is built by __graft_entry__.build()."""
import os
import subprocess

import numpy as np
import pytest
import torch

from synth import workloads as W
from tests.gpu_util import need_gpu, make_trace, trace_np

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "moe_q2_consumer")

CASES = [
    # the tiny fp32 layer (no shared expert, no bias); a bf16 layer with a shared expert,
    # a Zipf router bias and a ragged token count; the same under Q8 activations
    (W.WORKLOADS["tiny"], 0),
    (W.Workload("c_abi_e16", 61, 9, 512, 16, 4, 512, 256, "bf16", 0.05, zipf=True), 0),
    (W.Workload("c_abi_e16", 61, 9, 512, 16, 4, 512, 256, "bf16", 0.05, zipf=True), "ACT_Q8"),
]


@pytest.mark.parametrize("case", CASES, ids=["tiny", "bf16_shared_bias", "bf16_q8"])
def test_c_consumer_matches_binding(case, tmp_path):
    mq = need_gpu()
    if not os.path.exists(EXE):
        pytest.fail("tests/c/moe_q2_consumer is missing: run __graft_entry__.build() first")
    from bit_quantized_routed_amd import workload as dw
    wl, flag = case
    flags = getattr(mq, flag) if flag else 0
    dl = dw.DeviceLayer(wl)
    shape = dl.shape(flags)
    T, K, E, H = wl.tokens, wl.topk, wl.n_experts, wl.hidden
    x = dw.activations(wl)
    ws = dw.workspace(shape, T, K)
    out = torch.zeros((T, H), dtype=torch.float32, device="cuda")
    tr = make_trace(T, K, E)
    mq.forward(x, dl.router_w, dl.experts, dl.shared_w, K, out, shape, T, router_b=dl.router_b, workspace=ws,
               trace=tr)
    torch.cuda.synchronize()
    ref, ref_idx = out.cpu().numpy(), trace_np(tr)["topk_idx"]
    d = str(tmp_path)
    act = 1 if wl.act == "bf16" else 0
    with open(os.path.join(d, "meta.txt"), "w") as f:
        f.write("%d %d %d %d %d %d %d %d %r %d\n" % (H, wl.inter, E, K, wl.shared_inter, act, shape.flags, T,
                                                     float(shape.rms_eps), 1 if dl.router_b is not None else 0))
    def raw(t, name):                  # the tensor's bytes, whatever its dtype
        t.detach().cpu().contiguous().reshape(-1).view(torch.uint8).numpy().tofile(os.path.join(d, name))
    raw(x, "x.bin")
    raw(dl.router_w, "router_w.bin")
    raw(dl.experts, "experts.bin")
    if wl.shared_inter:
        raw(dl.shared_w, "shared.bin")
    if dl.router_b is not None:
        raw(dl.router_b, "router_b.bin")
    p = subprocess.run([EXE, d], capture_output=True, text=True, timeout=120)
    print(p.stdout, p.stderr)
    assert p.returncode == 0, p.stderr
    assert "topk 0: " in p.stdout and "no workspace: " in p.stdout
    got = np.fromfile(os.path.join(d, "out.bin"), dtype=np.float32).reshape(T, H)
    got_idx = np.fromfile(os.path.join(d, "idx.bin"), dtype=np.int32).reshape(T, K)
    assert np.array_equal(got, ref)
    assert np.array_equal(got_idx, ref_idx)

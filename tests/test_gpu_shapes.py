"""GPU parity on small, odd layer shapes: expert counts that leave a partial chunk of
64 in the top-K ranking, K = 1, K = E, the largest E and K the library accepts, fp32
and bf16 inputs, with and without a shared expert, Zipf-biased routing, token counts
on both sides of every launch-shape switch (routing inside the decode gate/up launch
up to 4 tokens and E <= 256, with its one-token shortcut; per-expert router up to 8;
decode kernels below 256 tokens; prefill kernels and the chunked bucketing from
256, also with E > 256; with more work items than work-groups and 3 or more block
columns, so that each item's successor is staged during it, and with units of 80 and
48 slots), and an empty batch.  Every token's routing and the bucketing are checked;
the outputs of every token outside the near-tie window are compared with the oracle."""
import numpy as np
import pytest
import torch

from oracle import moe
from synth import workloads as W
from tests.gpu_util import need_gpu, make_trace, trace_np, check_routing, rel_err
from tests.oracle_inputs import HostLayer

pytestmark = pytest.mark.gpu

TOL_DECODE = 2e-3
TOL_PREFILL = 2e-3          # the exact-integer prefill kernels (observed ~3e-4)

#        name         seed  T    H    E   K   I    Is   act     router sigma  zipf
CASES = [
    ("e100_k6_t5",    11,   5,  256, 100, 6, 256, 256, "bf16", 0.05, False),
    ("e65_k1_t3_f32", 12,   3,  512,  65, 1, 256,   0, "f32",  0.05, False),
    ("e16_k16_t9",    13,   9,  256,  16, 16, 512, 256, "bf16", 0.05, False),
    ("e300_k8_t40",   14,  40,  256, 300, 8, 256, 256, "bf16", 0.05, True),
    ("e512_k16_t2",   15,   2,  256, 512, 16, 256,   0, "bf16", 0.05, False),
    ("e8_k2_t300",    16, 300,  256,   8, 2, 512, 256, "bf16", 0.05, False),
    ("e33_k4_t1_f32", 17,   1,  256,  33, 4, 256, 256, "f32",  0.05, False),
    ("e16_k16_t1",    18,   1,  256,  16, 16, 256, 256, "bf16", 0.05, False),
    ("e300_k8_t260",  19, 260,  256, 300, 8, 256, 256, "bf16", 0.05, True),
    ("e64_k8_t1024",  20, 1024, 1536, 64, 8, 768, 256, "bf16", 0.05, False),
]


def _workload(case):
    name, seed, T, H, E, K, I, Is, act, rs, zipf = case
    return W.Workload(name, seed, T, H, E, K, I, Is, act, rs, zipf=zipf)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_shape(case):
    mq = need_gpu()
    from bit_quantized_routed_amd import workload as dw
    wl = _workload(case)
    T, K, E, H, I = wl.tokens, wl.topk, wl.n_experts, wl.hidden, wl.inter
    dl = dw.DeviceLayer(wl)
    hl = HostLayer(wl)
    eb = wl.expert_bytes
    dev_bytes = dl.experts.cpu().numpy()
    for e in sorted({0, E // 2, E - 1}):       # device encoder + packer = host oracle's
        assert np.array_equal(dev_bytes[e * eb:(e + 1) * eb], hl.packed_expert(e))
    x = dw.activations(wl)
    shape = dl.shape(0)
    ws = dw.workspace(shape, T, K)
    tr = make_trace(T, K, E)
    out = torch.zeros((T, H), dtype=torch.float32, device="cuda")
    mq.forward(x, dl.router_w, dl.experts, dl.shared_w, K, out, shape, T,
               router_b=dl.router_b, workspace=ws, trace=tr)
    torch.cuda.synchronize()
    out = out.cpu().numpy().astype(np.float64)
    tr = trace_np(tr)
    xh, _ = W.activations(wl)
    idx, g, logits, margin = moe.route(xh, hl.router_w, hl.router_b, K)
    excluded, rep = check_routing(tr, {"idx": idx, "g": g, "logits": logits, "margin": margin}, E, K)
    if K == 1:
        assert np.all(tr["topk_w"] == 1.0)
    toks = np.nonzero(~excluded)[0]
    assert toks.size > 0
    ref, _ = moe.layer(xh[toks], hl.router_w, hl.router_b, hl.expert_bytes, hl.shared, K, H, I)
    err = rel_err(out[toks], ref)
    tol = TOL_PREFILL if T >= 256 else TOL_DECODE
    print(case[0], rep, "tokens", toks.size, "rel_err", err)
    assert err <= tol


def test_empty_batch_leaves_output_untouched():
    mq = need_gpu()
    from bit_quantized_routed_amd import workload as dw
    wl = _workload(CASES[0])
    dl = dw.DeviceLayer(wl)
    shape = dl.shape(0)
    out = torch.full((1, wl.hidden), 7.0, dtype=torch.float32, device="cuda")
    x = dw.activations(wl)
    ws = dw.workspace(shape, 1, wl.topk)
    mq.forward(x, dl.router_w, dl.experts, dl.shared_w, wl.topk, out, shape, 0,
               router_b=dl.router_b, workspace=ws)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)


# the same odd shapes under the layer's options: batch invariance, Q8 activations,
# the 4-bit sibling format for all routed matrices, and all three together (Q8
# against the oracle's Q8 mode)
OPT_CASES = ["e100_k6_t5", "e65_k1_t3_f32", "e16_k16_t9", "e300_k8_t40", "e512_k16_t2", "e8_k2_t300",
             "e16_k16_t1"]
OPTIONS = {"bi": ("BATCH_INVARIANT",), "q8": ("ACT_Q8",), "q4": (), "bi_q8_q4": ("BATCH_INVARIANT", "ACT_Q8")}


@pytest.mark.parametrize("opt", list(OPTIONS))
@pytest.mark.parametrize("name", OPT_CASES)
def test_shape_options(name, opt):
    mq = need_gpu()
    from bit_quantized_routed_amd import workload as dw
    case = next(c for c in CASES if c[0] == name)
    _, seed, T, H, E, K, I, Is, act, rs, zipf = case
    q4 = opt in ("q4", "bi_q8_q4")
    wl = W.Workload(name + "_" + opt, seed, T, H, E, K, I, Is, act, rs, zipf=zipf, q4_gu=q4, q4_down=q4)
    dl = dw.DeviceLayer(wl)
    hl = HostLayer(wl)
    flags = 0
    for f in OPTIONS[opt]:
        flags |= getattr(mq, f)
    shape = dl.shape(flags)
    x = dw.activations(wl)
    ws = dw.workspace(shape, T, K)
    tr = make_trace(T, K, E)
    out = torch.zeros((T, H), dtype=torch.float32, device="cuda")
    mq.forward(x, dl.router_w, dl.experts, dl.shared_w, K, out, shape, T,
               router_b=dl.router_b, workspace=ws, trace=tr)
    torch.cuda.synchronize()
    out = out.cpu().numpy().astype(np.float64)
    tr = trace_np(tr)
    xh, _ = W.activations(wl)
    idx, g, logits, margin = moe.route(xh, hl.router_w, hl.router_b, K)
    excluded, rep = check_routing(tr, {"idx": idx, "g": g, "logits": logits, "margin": margin}, E, K)
    toks = np.nonzero(~excluded)[0]
    assert toks.size > 0
    a = "q8" if "ACT_Q8" in OPTIONS[opt] else "exact"
    ref, _ = moe.layer(xh[toks], hl.router_w, hl.router_b, hl.expert_bytes, hl.shared, K, H, I, act=a)
    err = rel_err(out[toks], ref)
    print(name, opt, rep, "tokens", toks.size, "rel_err", err)
    assert err <= TOL_DECODE

"""GPU parity of the layer's options against the oracle: the 4-bit sibling format
(whole experts and per-matrix mixes, at decode and prefill batch sizes), Q8
activations (decode and prefill kernels, the one-token path), and the
batch-invariant mode on the speculative-verification micro-batch (16 sessions x 6
tokens): a token's outputs, routing and gates are the same bits alone and inside
any batch."""
import functools

import numpy as np
import pytest
import torch

from oracle import moe
from synth import workloads as W
from tests.gpu_util import need_gpu, make_trace, trace_np, check_routing, rel_err, NEAR_TIE
from tests.oracle_inputs import HostLayer

pytestmark = pytest.mark.gpu

TOL = 2e-3
# Q8 against the oracle's Q8 mode: both sides quantise the layer input identically
# (exact); the SwiGLU output is quantised from fp32 values that differ by ~1e-6
# relative, so now and then one of its 2048 codes per slot lands one step apart
# (about 0.3 per slot at the decode shape), which moves that token's output by
# ~7e-4 of its maximum at most: the same 2e-3.
TOL_Q8 = 2e-3


def _layer(mq, dl, x, T, flags=0, out=None):
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


def _check(wl, out, tr, act="exact", toks=None, pooled=False, tol=TOL):
    """Routing of every token, bucketing, outputs of `toks` (default all) vs the oracle."""
    hl = HostLayer(wl)
    xh, _ = W.activations(wl)
    idx, g, logits, margin = moe.route(xh, hl.router_w, hl.router_b, wl.topk)
    excluded, rep = check_routing(tr, {"idx": idx, "g": g, "logits": logits, "margin": margin},
                                  wl.n_experts, wl.topk)
    toks = np.arange(wl.tokens) if toks is None else np.asarray(toks)
    toks = toks[~excluded[toks]]
    if pooled:
        ref = _pooled(wl.name, tuple(int(t) for t in toks), act)
    else:
        ref, _ = moe.layer(xh[toks], hl.router_w, hl.router_b, hl.expert_bytes, hl.shared, wl.topk,
                           wl.hidden, wl.inter, act=act)
    err = rel_err(out[toks], ref)
    print(wl.name, act, rep, "tokens compared", toks.size, "rel_err", err, flush=True)
    assert toks.size >= len(toks) - 2
    assert err <= tol
    return err, ref, toks


@functools.lru_cache(maxsize=8)
def _pooled(name, toks, act):
    from tests.oracle_pool import ExpertPool, layer_outputs
    wl = W.WORKLOADS[name]
    xh, _ = W.activations(wl)
    pool = ExpertPool()
    try:
        (ref, _), = layer_outputs(pool, name, [(0, HostLayer(wl), xh[list(toks)])], wl.topk, wl.hidden,
                                  wl.inter, act=act)
    finally:
        pool.close()
    return ref


# ------------------------------------------------------------------ 4-bit sibling
Q4_CASES = [
    # name          seed T    H    E   K  I    Is   act     q4_gu q4_down
    ("q4_t5",        31, 5,   256, 8,  2, 512, 256, "bf16", True, True),
    ("q4dn_t3_f32",  32, 3,   512, 16, 4, 256, 0,   "f32",  False, True),
    ("q4gu_t40",     33, 40,  256, 65, 8, 256, 256, "bf16", True, False),
    ("q4_t300",      34, 300, 256, 8,  2, 512, 256, "bf16", True, True),   # prefill kernels at 300 tokens
    ("q4_t1_k16",    35, 1,   256, 16, 16, 256, 256, "bf16", True, True),  # one token, in-launch routing
]


@pytest.mark.parametrize("case", Q4_CASES, ids=[c[0] for c in Q4_CASES])
def test_q4_formats(case):
    mq = need_gpu()
    from bit_quantized_routed_amd import workload as dw
    name, seed, T, H, E, K, I, Is, act, gu, dn = case
    wl = W.Workload(name, seed, T, H, E, K, I, Is, act, 0.05, q4_gu=gu, q4_down=dn)
    dl = dw.DeviceLayer(wl)
    hl = HostLayer(wl)
    eb = wl.expert_bytes
    dev = dl.experts.cpu().numpy()
    for e in sorted({0, E - 1}):                  # device encoders + packer = the oracle's
        assert np.array_equal(dev[e * eb:(e + 1) * eb], hl.packed_expert(e))
    plan = mq.describe(dl.shape(0), T, K)
    assert plan["path"] == (mq.PATH_PREFILL if T >= mq.PREFILL_MIN_TOKENS else mq.PATH_DECODE)
    out, tr = _layer(mq, dl, dw.activations(wl), T)
    _check(wl, out, tr)


Q4_PREFILL_CASES = [
    # name            seed T    H     E   K  I    Is   act     q4_gu q4_down flags
    # 64-slot units, several per expert with a ragged last one; more work items than
    # work-groups; 4 and 3 block columns (chained items)
    ("q4pf_t600",      36, 600, 1024, 16, 4, 768, 0,   "bf16", True,  True,  ()),
    # one 4-bit matrix: the 2-bit matrix's launch also on 64-slot units
    ("q4gupf_t300",    37, 300, 512,  16, 4, 512, 256, "bf16", True,  False, ()),
    ("q4dnpf_t40",     38, 40,  512,  16, 8, 768, 0,   "f32",  False, True,  ("PATH_PREFILL",)),
    # Q8 activations: 80-slot units for both formats
    ("q4pf_q8_t600",   39, 600, 1024, 16, 4, 768, 0,   "bf16", True,  True,  ("ACT_Q8",)),
    ("q4gupf_q8_t64",  40, 64,  512,  65, 8, 256, 256, "bf16", True,  False, ("ACT_Q8", "PATH_PREFILL")),
]


@pytest.mark.parametrize("case", Q4_PREFILL_CASES, ids=[c[0] for c in Q4_PREFILL_CASES])
def test_q4_prefill(case):
    """The prefill kernels on the 4-bit format (both matrices, and either one), with
    the default two-digit and with Q8 activations, against the oracle."""
    mq = need_gpu()
    from bit_quantized_routed_amd import workload as dw
    name, seed, T, H, E, K, I, Is, act, gu, dn, names = case
    wl = W.Workload(name, seed, T, H, E, K, I, Is, act, 0.05, q4_gu=gu, q4_down=dn)
    dl = dw.DeviceLayer(wl)
    f = 0
    for n in names:
        f |= getattr(mq, n)
    assert mq.describe(dl.shape(f), T, K)["routed_kernel"] == 2
    out, tr = _layer(mq, dl, dw.activations(wl), T, flags=f)
    q8 = "ACT_Q8" in names
    _check(wl, out, tr, act="q8" if q8 else "exact", tol=TOL_Q8 if q8 else TOL)


@pytest.mark.parametrize("flag", ["", "ACT_Q8"])
def test_decode1_q4(flag):
    """The full-size one-token layer at Q4 (in-launch routing, the down launch's own
    activation preparation and the shared rows in the routed launches, with 148-byte
    blocks), default and Q8 activations, against the oracle."""
    mq = need_gpu()
    from bit_quantized_routed_amd import workload as dw
    wl = W.WORKLOADS["decode1_q4"]
    dl = dw.DeviceLayer(wl)
    f = getattr(mq, flag) if flag else 0
    plan = mq.describe(dl.shape(f), 1, wl.topk)
    assert plan["path"] == mq.PATH_DECODE and plan["shared_fused"] == 1
    out, tr = _layer(mq, dl, dw.activations(wl), 1, flags=f)
    q8 = flag == "ACT_Q8"
    _check(wl, out, tr, act="q8" if q8 else "exact", pooled=True, tol=TOL_Q8 if q8 else TOL)


def test_tiny_q4_workloads():
    mq = need_gpu()
    from bit_quantized_routed_amd import workload as dw
    for name in ("tiny_q4", "tiny_q4gu"):
        wl = W.WORKLOADS[name]
        dl = dw.DeviceLayer(wl)
        assert np.array_equal(dl.experts.cpu().numpy(), HostLayer(wl).all_expert_bytes())
        out, tr = _layer(mq, dl, dw.activations(wl), wl.tokens)
        _check(wl, out, tr)


def test_stack40_q2q4_q4_layers():
    """The 4-bit layers (34..39) of the q2-q4 stack, each on its own residual input at
    full size (RMSNorm -> layer -> residual add), 4 tokens each through the oracle."""
    mq = need_gpu()
    from bit_quantized_routed_amd import workload as dw
    from tests.oracle_pool import ExpertPool, layer_outputs
    from tests.test_gpu_prefill_stack import _shared_sample
    wl = W.WORKLOADS["stack40_q2q4"]
    T, K, E = wl.tokens, wl.topk, wl.n_experts
    jobs, incs = [], []
    tmp = torch.empty(wl.hidden * wl.inter, dtype=torch.float32, device="cuda")
    for l in (33, 34, 39):                        # the last 2-bit layer and two 4-bit ones
        dl = dw.DeviceLayer(wl, layer=l, tmp=tmp)
        assert dl.codec_flags == (0 if l < 34 else mq.GU_Q4 | mq.DOWN_Q4)
        h = dw.layer_residual(wl, l)
        h_in = h.clone()
        shape = dl.shape(mq.RESIDUAL_ADD)
        ws = dw.workspace(shape, T, K)
        tr = make_trace(T, K, E)
        mq.forward(h, dl.router_w, dl.experts, dl.shared_w, K, h, shape, T, router_b=dl.router_b,
                   workspace=ws, trace=tr)
        torch.cuda.synchronize()
        inc = h.cpu().numpy().astype(np.float64) - h_in.cpu().numpy().astype(np.float64)
        trn = trace_np(tr)
        del dl, ws, h, h_in
        hl = HostLayer(wl, l)
        xl = moe.rmsnorm_bf16(W.layer_residual(wl, l), wl.rms_eps)
        idx, g, logits, margin = moe.route(xl, hl.router_w, hl.router_b, K)
        excluded, rep = check_routing(trn, {"idx": idx, "g": g, "logits": logits, "margin": margin}, E, K)
        toks = _shared_sample(idx, excluded, T - 1, 4)
        jobs.append((l, hl, xl[toks]))
        incs.append(inc[toks])
        print("  [q2q4] layer %d done, %s, tokens %s" % (l, rep, toks), flush=True)
    del tmp
    pool = ExpertPool()
    try:
        refs = layer_outputs(pool, wl.name, jobs, K, wl.hidden, wl.inter)
    finally:
        pool.close()
    errs = [rel_err(i, r) for i, (r, _) in zip(incs, refs)]
    print("stack40_q2q4 layers 33, 34, 39 rel_err", errs)
    assert max(errs) <= TOL


# ------------------------------------------------------------------ Q8 activations
@pytest.mark.parametrize("name,flag", [("tiny", ""), ("tiny", "PATH_PREFILL"), ("tiny_q4", ""),
                                       ("decode1", ""), ("decode32_zipf", ""),
                                       ("decode32_zipf", "PATH_PREFILL")])
def test_q8_activations(name, flag):
    """Q8 activations on the decode kernels (one token: the down launch's own
    preparation; micro-batch), the prefill kernels and the 4-bit format, against the
    oracle's Q8 mode; the distance to the exact layer is reported."""
    mq = need_gpu()
    from bit_quantized_routed_amd import workload as dw
    wl = W.WORKLOADS[name]
    dl = dw.DeviceLayer(wl)
    f = mq.ACT_Q8 | (getattr(mq, flag) if flag else 0)
    out, tr = _layer(mq, dl, dw.activations(wl), wl.tokens, flags=f)
    big = wl.hidden > 1024
    err, _, toks = _check(wl, out, tr, act="q8", pooled=big, tol=TOL_Q8)
    if not big:
        _, ref_exact, _ = _check(wl, out, tr, act="exact", toks=toks, tol=1.0)
        print("  Q8 layer against the exact layer:", rel_err(out[toks], ref_exact))


def test_q8_prefill_many_items():
    """Q8 on the prefill kernels with more work items than work-groups and chained
    items (1024 tokens, 64 experts, 6 and 3 block columns)."""
    mq = need_gpu()
    from bit_quantized_routed_amd import workload as dw
    wl = W.Workload("q8_e64_t1024", 21, 1024, 1536, 64, 8, 768, 256, "bf16", 0.05)
    dl = dw.DeviceLayer(wl)
    assert mq.describe(dl.shape(mq.ACT_Q8), wl.tokens, wl.topk)["routed_kernel"] == 2
    out, tr = _layer(mq, dl, dw.activations(wl), wl.tokens, flags=mq.ACT_Q8)
    _check(wl, out, tr, act="q8", tol=TOL_Q8)


# ------------------------------------------------------------------ verification micro-batch
def test_verify96_parity():
    """The 96-token verification micro-batch, default flags and batch-invariant, all
    tokens against the oracle."""
    mq = need_gpu()
    from bit_quantized_routed_amd import workload as dw
    wl = W.WORKLOADS["verify96_zipf"]
    dl = dw.DeviceLayer(wl)
    x = dw.activations(wl)
    for f in (0, mq.BATCH_INVARIANT):
        out, tr = _layer(mq, dl, x, wl.tokens, flags=f)
        _check(wl, out, tr, pooled=True)


def test_batch_invariance():
    """Under MOE_Q2_BATCH_INVARIANT a token's output, routing and gates are the same
    bits alone (1 token), in its session's 6, in the 96-token micro-batch and in a
    300-token batch (prefill size, still the decode kernels).  Without the flag the
    same comparison is bounded: split counts and router formulation change with the
    batch size, so fp32 sums round differently (relative deviation <= 1e-5 outside
    near ties)."""
    mq = need_gpu()
    from bit_quantized_routed_amd import workload as dw
    wl = W.WORKLOADS["verify96_zipf"]
    dl = dw.DeviceLayer(wl)
    x300 = dw.activations(wl, tokens=300)
    assert torch.equal(x300[:96], dw.activations(wl))
    sample = [0, 5, 6, 47, 95]
    xh, _ = W.activations(wl)
    hl = HostLayer(wl)
    _, _, _, margin = moe.route(xh, hl.router_w, hl.router_b, wl.topk)
    for f, exact in ((mq.BATCH_INVARIANT, True), (0, False)):
        batches = {}
        for T in (96, 300):
            batches[T] = _layer(mq, dl, x300[:T].contiguous(), T, flags=f)
        worst = 0.0
        for t in sample:
            s0 = 6 * (t // 6)
            alone = _layer(mq, dl, x300[t:t + 1].contiguous(), 1, flags=f)
            session = _layer(mq, dl, x300[s0:s0 + 6].contiguous(), 6, flags=f)
            views = [(alone[0][0], alone[1]["topk_idx"][0], alone[1]["topk_w"][0]),
                     (session[0][t - s0], session[1]["topk_idx"][t - s0], session[1]["topk_w"][t - s0])]
            views += [(o[t], tr["topk_idx"][t], tr["topk_w"][t]) for o, tr in batches.values()]
            for o, i, g in views[1:]:
                if exact:
                    assert np.array_equal(o, views[0][0]), (t, "output")
                    assert np.array_equal(i, views[0][1]) and np.array_equal(g, views[0][2]), (t, "routing")
                elif margin[t] >= NEAR_TIE:
                    worst = max(worst, float(np.abs(o - views[0][0]).max() / np.abs(views[0][0]).max()))
        if not exact:
            print("  default flags: largest relative deviation of a token between batches", worst)
            assert worst <= 1e-5

"""Helpers of the GPU parity tests: run the HIP layer through the C ABI and
compare with the oracle under the parity rules.

Rules: routing must agree as sets for every token whose oracle margin
l_(K) - l_(K+1) is at least 1e-4 (near-tie tokens are counted, and their GPU
selection must still be a valid top-K up to that margin); bucketing must equal
the stable bucketing of the GPU's own routing exactly; outputs are compared per
token with the infinity-norm relative error max|o - r| / max|r|."""
import numpy as np
import pytest
import torch

from oracle import moe

NEAR_TIE = 1e-4
# Gate weights: fp32 logits (error ~1e-6 at H = 7168) through an fp32 softmax; the
# derivative of a renormalised gate with respect to a logit is at most 1/4.
GATE_TOL = 1e-5


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_quantized_routed_amd as mq
    mq.library()          # raises if the HIP library is missing
    return mq


def make_trace(T, K, E):
    dev = "cuda"
    return dict(topk_idx=torch.full((T, K), -1, dtype=torch.int32, device=dev),
                topk_w=torch.zeros((T, K), dtype=torch.float32, device=dev),
                counts=torch.full((E,), -1, dtype=torch.int32, device=dev),
                offsets=torch.full((E + 1,), -1, dtype=torch.int32, device=dev),
                perm=torch.full((T * K,), -1, dtype=torch.int32, device=dev))


def trace_np(tr):
    return {k: v.cpu().numpy() for k, v in tr.items()}


def check_routing(tr, route, E, K):
    """Returns (excluded mask, report).  Asserts set equality outside near ties,
    validity inside them, the descending order of the selection wherever the
    oracle's order is not itself a near tie, gate weights within GATE_TOL, and exact
    bucketing: against the oracle's own routing when no token is a near tie, else
    against the stable bucketing of the GPU routing."""
    idx = tr["topk_idx"]
    ref = route["idx"]
    logits = route["logits"]
    margin = route["margin"]
    T = idx.shape[0]
    excluded = margin < NEAR_TIE
    ordered = 0
    for t in range(T):
        if excluded[t]:
            kth = np.sort(logits[t])[::-1][K - 1]
            assert np.all(logits[t, idx[t]] >= kth - NEAR_TIE), t
            assert len(set(idx[t].tolist())) == K
        else:
            assert set(idx[t].tolist()) == set(ref[t].tolist()), (t, idx[t], ref[t])
            # order of the selection: descending logit where the gaps are resolvable
            gaps = -np.diff(logits[t, ref[t]])
            if K == 1 or gaps.min() >= NEAR_TIE:
                assert idx[t].tolist() == ref[t].tolist(), (t, idx[t], ref[t])
                ordered += 1
    if not excluded.any() and ordered == T:
        counts, offsets, perm, _ = moe.bucket(ref, E)     # the oracle's routing, bucketed
    else:
        counts, offsets, perm, _ = moe.bucket(idx, E)     # valid alternatives: the GPU's
    assert np.array_equal(tr["counts"], counts)
    assert np.array_equal(tr["offsets"], offsets)
    assert np.array_equal(tr["perm"], perm)
    # gates: compare per expert for agreeing tokens
    gmax = 0.0
    for t in range(T):
        if excluded[t]:
            continue
        a = dict(zip(idx[t].tolist(), tr["topk_w"][t].tolist()))
        b = dict(zip(ref[t].tolist(), route["g"][t].tolist()))
        for e in a:
            gmax = max(gmax, abs(a[e] - b[e]))
    assert gmax <= GATE_TOL, gmax
    assert abs(tr["topk_w"].sum(axis=1) - 1).max() < 1e-5
    return excluded, {"excluded": int(excluded.sum()), "ordered": ordered, "gate_abs_err": gmax}


def rel_err(out, ref, mask=None):
    num = np.abs(out - ref).max(axis=1)
    den = np.abs(ref).max(axis=1)
    r = num / np.maximum(den, 1e-300)
    if mask is not None:
        r = r[mask]
    return float(r.max()) if r.size else 0.0

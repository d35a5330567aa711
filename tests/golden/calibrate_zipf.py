"""Calibrate the router-bias strength alpha of the Zipf workloads.

The micro-batched decode workloads bias the router so that expert popularity
follows Zipf(s = 1.1): b_e = -alpha * ln(r_e) is added to every logit, with r_e a
seeded popularity rank.  Exact Zipf slot shares are infeasible for top-8 of 256
(K * p_1 > 1), so alpha is chosen such that the least-squares slope of
log(selection frequency) against log(rank), over ranks 10..200, equals -1.1.

Selection frequencies come from the oracle's router on a calibration batch
(router N(0, 0.02^2), activations N(0, 1) rounded to bf16, dedicated seed).
Writes synth/zipf_alpha.json.  Run:  python tests/golden/calibrate_zipf.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import moe  # noqa: E402
from synth import workloads as W  # noqa: E402

CAL_SEED = 1000
CAL_TOKENS = 20000
TARGET_SLOPE = -1.1


def slope_for(alpha, logits, rank, topk):
    b = -alpha * np.log(rank.astype(np.float64))
    l = logits + b[None, :]
    sel = np.argpartition(-l, topk, axis=1)[:, :topk]
    freq = np.bincount(rank[sel.reshape(-1)], minlength=rank.size + 1)[1:].astype(np.float64)
    r = np.arange(1, rank.size + 1)
    m = (r >= 10) & (r <= 200) & (freq > 0)
    A = np.vstack([np.log(r[m]), np.ones(m.sum())]).T
    return np.linalg.lstsq(A, np.log(freq[m]), rcond=None)[0][0]


def main():
    base = W.WORKLOADS["decode32_zipf"]
    wl = W.Workload("cal", CAL_SEED, CAL_TOKENS, base.hidden, base.n_experts, base.topk,
                    base.inter, base.shared_inter, "bf16", base.router_sigma, zipf=True)
    x, _ = W.activations(wl)
    Wr = W.router_weights(wl)
    _, _, logits, _ = moe.route(x, Wr, None, wl.topk)
    rank = W.router_rank(wl)
    lo, hi = 0.3, 1.5
    for _ in range(40):
        mid = 0.5 * (lo + hi)
        if slope_for(mid, logits, rank, wl.topk) > TARGET_SLOPE:
            lo = mid
        else:
            hi = mid
    alpha = round(0.5 * (lo + hi), 4)
    s = slope_for(alpha, logits, rank, wl.topk)
    out = {"alpha": alpha, "slope": round(float(s), 4), "target_slope": TARGET_SLOPE,
           "calibration_seed": CAL_SEED, "calibration_tokens": CAL_TOKENS,
           "ranks": [10, 200], "script": "tests/golden/calibrate_zipf.py"}
    with open(os.path.join(ROOT, "synth", "zipf_alpha.json"), "w") as f:
        json.dump(out, f, indent=1)
    print(out)


if __name__ == "__main__":
    main()

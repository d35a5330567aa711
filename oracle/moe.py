"""Routed-expert MoE layer, oracle side (plain NumPy, fp64).

TEST INFRASTRUCTURE: only tests/, the smoke check and the benchmark's CPU
baseline may import this package.  It shares no code with the HIP library.

What the layer computes (ds4 README mirror, section "Model Weights": only the
routed MoE experts are 2-bit; shared experts, projections and routing stay at
full precision; DeepSeek-style layer: softmax router, top-K experts with the
selected probabilities renormalised, SwiGLU expert FFNs, one shared expert):

    l_t      = x_t . Wr^T (+ b)                       router logits, fp64
    S_t      = the K largest l_t,e (ties: lower e first), descending
    g_t,k    = softmax(l_t)[S_t,k] / sum_{j in S_t} softmax(l_t)[j]
    FFN_e(x) = (silu(x . Wg_e^T) * (x . Wu_e^T)) . Wd_e^T,  silu(a) = a / (1 + e^-a)
    out_t    = FFN_shared(x_t) + sum_k g_t,k * FFN_{S_t,k}(x_t)

and, for a stack of layers with a residual stream h (fp32) and RMSNorm:

    x_l     = bf16_rne(h_l / sqrt(mean(h_l^2) + eps))
    h_{l+1} = h_l + layer_l(x_l)

Expert weights come from their block bytes through q2.decode_* (the 2-bit
format) or q4.decode_* (its 4-bit sibling), chosen per matrix by the block size;
every product and sum after that is fp64.

Q8 activation mode (act="q8"; ds4 README mirror, section "Model Weights": decode
uses Q8 activations): the routed experts' two inputs -- the layer input x and the
SwiGLU output h -- are replaced by their per-row Q8 values before the products,
see q8_rows.  Router and shared expert stay at full precision.
"""
import numpy as np

from . import q2, q4


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def route(x, router_w, router_b, topk):
    """Router logits, top-K selection and renormalised gate weights.

    Returns idx [T, K] int32 (descending logit, ties to the lower expert index),
    g [T, K] fp64, logits [T, E] fp64 and margin [T] = l_(K) - l_(K+1) on the
    sorted row (inf when K equals the expert count)."""
    x = _f64(x)
    W = _f64(router_w)
    logits = x @ W.T
    if router_b is not None:
        logits = logits + _f64(router_b)[None, :]
    T, E = logits.shape
    order = np.argsort(-logits, axis=1, kind="stable")
    idx = order[:, :topk].astype(np.int32)
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    p = p / p.sum(axis=1, keepdims=True)
    sel = np.take_along_axis(p, idx.astype(np.int64), axis=1)
    g = sel / sel.sum(axis=1, keepdims=True)
    srt = np.take_along_axis(logits, order, axis=1)
    if topk < E:
        margin = srt[:, topk - 1] - srt[:, topk]
    else:
        margin = np.full(T, np.inf)
    return idx, g, logits, margin


def bucket(idx, n_experts):
    """Token-by-expert bucketing of the slots s = t*K + k.

    counts[e]  = number of slots routed to e        (histogram)
    offsets    = [0, cumsum(counts)]                 (exclusive scan, E+1 entries)
    perm[p]    = slot at bucket position p, ordered by (expert, token)  (stable)
    inv[s]     = bucket position of slot s"""
    e = np.asarray(idx, dtype=np.int64).reshape(-1)
    counts = np.bincount(e, minlength=n_experts).astype(np.int32)
    offsets = np.zeros(n_experts + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    perm = np.argsort(e, kind="stable").astype(np.int32)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size, dtype=np.int32)
    return counts, offsets, perm, inv


def silu(a):
    with np.errstate(over="ignore"):
        return a / (1.0 + np.exp(-a))


def q8_rows(v):
    """Q8 activations of rows v [n, L] (values as fp64): per row, with max|v| in
    [2^(e-1), 2^e), s = 2^(e - 7) and a = clamp(rint_even(v / s), -127, 127); returns
    a * s (exact in fp64).  The scale is a power of two, so v / s is exact and the
    rounding is a function of v alone; an all-zero row stays zero."""
    v = _f64(v)
    amax = np.abs(v).max(axis=1, keepdims=True)
    _, e = np.frexp(amax)
    s = np.ldexp(1.0, e - 7)
    a = np.clip(np.rint(v / s), -127, 127)
    return np.where(amax > 0, a * s, 0.0)


def ffn(x, w_gate, w_up, w_down, act="exact"):
    """SwiGLU FFN on token rows x [n, H]: (silu(x Wg^T) * (x Wu^T)) Wd^T, fp64.
    act="q8": x and h replaced by q8_rows of themselves (h rounded to fp32 first,
    the precision the rounding decision is taken in)."""
    x = _f64(x)
    if act == "q8":
        x = q8_rows(x)
    a = x @ _f64(w_gate).T
    c = x @ _f64(w_up).T
    h = silu(a) * c
    if act == "q8":
        h = q8_rows(h.astype(np.float32))
    return h @ _f64(w_down).T


def decode_matrix(raw, rows, cols):
    """Block bytes [n, 84] (2-bit format) or [n, 148] (Q4 sibling) -> fp32 [rows, cols]."""
    raw = np.asarray(raw, np.uint8)
    codec = {q2.BLOCK_BYTES: q2, q4.BLOCK_BYTES: q4}[raw.shape[-1]]
    return codec.decode_matrix(raw, rows, cols)


def expert_weights(raw_gate, raw_up, raw_down, hidden, inter):
    """Block bytes of one routed expert -> fp32 matrices (gate [I,H], up [I,H], down [H,I]),
    each matrix in the format its block size names."""
    return (decode_matrix(raw_gate, inter, hidden),
            decode_matrix(raw_up, inter, hidden),
            decode_matrix(raw_down, hidden, inter))


def layer(x, router_w, router_b, expert_bytes, shared, topk, hidden, inter, ffn_map=None, act="exact"):
    """One MoE layer in fp64.

    x            [T, H] activations (fp32 values, or bf16 values widened)
    expert_bytes callable e -> (gate, up, down) Q2 bytes of routed expert e
    shared       None, or (Wg [Is,H], Wu [Is,H], Wd [H,Is]) full-precision weights
    ffn_map      optional evaluator of the routed FFNs: called with a list of
                 (expert, token rows [n, H]) and returning the list of FFN outputs;
                 by default each is ffn(rows, *expert_weights(*expert_bytes(e)), act).
    act          "exact" or "q8": the routed experts' activation mode (see ffn)
    Returns out [T, H] fp64 and the routing dict."""
    x = _f64(x)
    idx, g, logits, margin = route(x, router_w, router_b, topk)
    out = np.zeros((x.shape[0], hidden), dtype=np.float64)
    if shared is not None:
        out += ffn(x, *shared)
    # Each (token, expert) pair is an independent FFN evaluation; evaluating all
    # tokens of one expert together only shares the decoded weights.
    work = []
    for e in np.unique(idx):
        toks, ks = np.nonzero(idx == e)
        work.append((int(e), toks, ks))
    if ffn_map is None:
        ys = [ffn(x[toks], *expert_weights(*expert_bytes(e), hidden, inter), act=act) for e, toks, _ in work]
    else:
        ys = ffn_map([(e, x[toks]) for e, toks, _ in work])
    for (e, toks, ks), y in zip(work, ys):
        out[toks] += g[toks, ks][:, None] * y
    return out, {"idx": idx, "g": g, "logits": logits, "margin": margin}


def rmsnorm_bf16(h, eps):
    """bf16_rne(h / sqrt(mean(h^2) + eps)) per row, unit gain; returns the bf16
    values as fp64."""
    h = _f64(h)
    y = h / np.sqrt(np.mean(h * h, axis=1, keepdims=True) + eps)
    return _round_bf16(y)


def _round_bf16(y):
    """Round fp64 values to the nearest bf16 value (ties to even), exactly.

    bf16 keeps 8 significant bits: for |y| in [2^(e-1), 2^e) the spacing is
    2^(e-8); below the smallest normal (2^-126) it is 2^-133.  y / spacing is
    exact in fp64, so one rint (ties to even) gives the correctly rounded value."""
    y = _f64(y)
    _, e = np.frexp(y)
    e = np.maximum(e, -125)
    ulp = np.ldexp(1.0, e - 8)
    return np.rint(y / ulp) * ulp


def stack(h0, layers, topk, hidden, inter, eps):
    """Residual stack: h_{l+1} = h_l + layer_l(rmsnorm_bf16(h_l)).

    layers: list of dicts with router_w, router_b, expert_bytes, shared and
    optionally ffn_map and act (see layer()).
    Returns the final residual stream [T, H] fp64 and per-layer routings."""
    h = _f64(h0)
    routings = []
    for L in layers:
        x = rmsnorm_bf16(h, eps)
        y, r = layer(x, L["router_w"], L["router_b"], L["expert_bytes"], L["shared"],
                     topk, hidden, inter, ffn_map=L.get("ffn_map"), act=L.get("act", "exact"))
        h = h + y
        routings.append(r)
    return h, routings

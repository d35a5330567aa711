"""Pins of the oracle's MoE layer: brute force on tiny inputs, closed forms,
special cases that reduce to a dense mixture, and exact invariants (no GPU)."""
import math

import numpy as np
import pytest

from oracle import moe, q2
from tests.oracle_inputs import host_layer
from synth import workloads as W


# ----------------------------------------------------------------- routing
def _route_bruteforce(logits, K):
    T, E = logits.shape
    idx, g = [], []
    for t in range(T):
        pairs = sorted(((-logits[t, e], e) for e in range(E)))
        sel = [e for _, e in pairs[:K]]
        mx = max(logits[t])
        p = [math.exp(logits[t, e] - mx) for e in range(E)]
        z = sum(p)
        p = [v / z for v in p]
        zs = sum(p[e] for e in sel)
        idx.append(sel)
        g.append([p[e] / zs for e in sel])
    return np.array(idx), np.array(g)


def test_route_matches_bruteforce():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 32))
    Wr = rng.standard_normal((9, 32)) * 0.3
    b = rng.standard_normal(9) * 0.1
    for K in (1, 2, 3, 9):
        idx, g, logits, margin = moe.route(x, Wr, b, K)
        bi, bg = _route_bruteforce(x @ Wr.T + b, K)
        assert np.array_equal(idx, bi)
        assert np.allclose(g, bg, rtol=0, atol=1e-14)
        assert np.allclose(g.sum(axis=1), 1.0, rtol=0, atol=1e-12)
        if K < 9:
            srt = np.sort(logits, axis=1)[:, ::-1]
            assert np.allclose(margin, srt[:, K - 1] - srt[:, K])
        else:
            assert np.all(np.isinf(margin))


def test_route_k1_and_k_equals_e():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 16))
    Wr = rng.standard_normal((6, 16))
    _, g, _, _ = moe.route(x, Wr, None, 1)
    assert np.all(g == 1.0)
    idx, g, logits, _ = moe.route(x, Wr, None, 6)
    full = np.exp(logits - logits.max(axis=1, keepdims=True))
    full /= full.sum(axis=1, keepdims=True)
    assert np.allclose(np.take_along_axis(full, idx.astype(np.int64), axis=1), g, atol=1e-15)


def test_route_ties_go_to_lower_index():
    x = np.ones((1, 4))
    Wr = np.array([[1, 0, 0, 0], [0, 0, 0, 1], [1, 0, 0, 0], [0, 1, 0, 0], [0, 0, 1, 0.0]])
    idx, g, _, margin = moe.route(x, Wr, None, 2)
    assert idx.tolist() == [[0, 1]]          # all logits equal to 1: lowest indices
    assert margin[0] == 0.0
    assert np.allclose(g, 0.5)


def test_route_bias_enters_gates():
    x = np.zeros((1, 4))
    Wr = np.zeros((3, 4))
    b = np.array([0.0, math.log(3.0), -5.0])
    idx, g, _, _ = moe.route(x, Wr, b, 2)
    assert idx.tolist() == [[1, 0]]
    assert np.allclose(g, [[0.75, 0.25]], atol=1e-15)


# ----------------------------------------------------------------- bucketing
def test_bucket_matches_loops():
    rng = np.random.default_rng(2)
    T, K, E = 37, 4, 11
    idx = np.array([rng.choice(E, K, replace=False) for _ in range(T)])
    counts, offsets, perm, inv = moe.bucket(idx, E)
    flat = idx.reshape(-1)
    want_perm = [s for e in range(E) for s in range(T * K) if flat[s] == e]
    assert perm.tolist() == want_perm
    assert counts.tolist() == [int((flat == e).sum()) for e in range(E)]
    assert offsets[0] == 0 and offsets[-1] == T * K
    assert np.all(offsets[1:] - offsets[:-1] == counts)
    assert np.array_equal(perm[inv], np.arange(T * K))


# ----------------------------------------------------------------- FFN closed form
def _onehot_q2(rows, cols, colmap, value):
    """Q2 bytes of a [rows, cols] matrix with one nonzero per row: W[r, colmap[r]] = value.
    value = d * sc * q with d = value / 3, sc = 1, q = 3 (exact); all mins 0."""
    raw = np.zeros((rows, cols // 256, 84), dtype=np.uint8)
    d16 = np.float16(value / 3)
    assert float(d16) * 3 == value
    for r in range(rows):
        c = colmap[r]
        blk = raw[r, c // 256]
        i = c % 256
        blk[i // 16] = 1                              # sc_j = 1, m_j = 0
        blk[16 + i // 4] |= 3 << (2 * (i % 4))
        blk[80:82] = np.frombuffer(d16.tobytes(), dtype=np.uint8)
    for r in range(rows):                             # d on the other blocks of the row too
        for b in range(cols // 256):
            raw[r, b, 80:82] = np.frombuffer(d16.tobytes(), dtype=np.uint8)
    return raw.reshape(-1, 84)


def test_ffn_closed_form_permutations():
    # H = 256, I = 512: gate row i reads x[pg(i)] * 0.75, up row i reads x[pu(i)] * 1.5,
    # down row k reads h[pd(k)] * 0.375.  y_k = 0.375 * silu(0.75 x[pg(j)]) * 1.5 x[pu(j)],
    # j = pd(k): the gate gets the SiLU, the up the linear term, both read x along H.
    H, I = 256, 512
    rng = np.random.default_rng(3)
    pg = rng.integers(0, H, I)
    pu = rng.integers(0, H, I)
    pd = rng.permutation(I)[:H]
    raw = (_onehot_q2(I, H, pg, 0.75), _onehot_q2(I, H, pu, 1.5), _onehot_q2(H, I, pd, 0.375))
    x = rng.standard_normal((3, H))
    wg, wu, wd = moe.expert_weights(*raw, H, I)
    y = moe.ffn(x, wg, wu, wd)
    for t in range(3):
        for k in range(H):
            j = pd[k]
            a = 0.75 * x[t, pg[j]]
            want = 0.375 * (a / (1 + math.exp(-a))) * 1.5 * x[t, pu[j]]
            assert abs(y[t, k] - want) <= 1e-14 * max(1.0, abs(want))


def test_silu_values():
    assert moe.silu(np.array([0.0]))[0] == 0.0
    assert abs(moe.silu(np.array([1.0]))[0] - 1 / (1 + math.exp(-1))) < 1e-16
    assert moe.silu(np.array([-1000.0]))[0] == 0.0
    assert moe.silu(np.array([1000.0]))[0] == 1000.0


# ----------------------------------------------------------------- layer identities
def _tiny():
    return host_layer("tiny")


def test_k_equals_e_is_dense_mixture():
    L = _tiny()
    wl = L.wl
    x, _ = W.activations(wl)
    E, H, I = wl.n_experts, wl.hidden, wl.inter
    out, r = moe.layer(x, L.router_w, None, L.expert_bytes, None, E, H, I)
    # independent path: stack all experts, einsum over e
    Wg = np.stack([q2.decode_matrix(L.expert_bytes(e)[0], I, H) for e in range(E)]).astype(np.float64)
    Wu = np.stack([q2.decode_matrix(L.expert_bytes(e)[1], I, H) for e in range(E)]).astype(np.float64)
    Wd = np.stack([q2.decode_matrix(L.expert_bytes(e)[2], H, I) for e in range(E)]).astype(np.float64)
    lg = x.astype(np.float64) @ L.router_w.astype(np.float64).T
    p = np.exp(lg - lg.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    a = np.einsum("th,eih->tei", x.astype(np.float64), Wg)
    c = np.einsum("th,eih->tei", x.astype(np.float64), Wu)
    h = a / (1 + np.exp(-a)) * c
    y = np.einsum("tei,ehi->teh", h, Wd)
    want = np.einsum("te,teh->th", p, y)
    assert np.allclose(out, want, rtol=0, atol=1e-12 * np.abs(want).max())


def test_single_expert_with_shared_is_sum():
    L = _tiny()
    wl = L.wl
    x, _ = W.activations(wl)
    H, I = wl.hidden, wl.inter
    one = L.expert_bytes(3)
    Wr = np.zeros((1, H))
    rng = np.random.default_rng(4)
    shared = (rng.standard_normal((I, H)) * 0.02, rng.standard_normal((I, H)) * 0.02,
              rng.standard_normal((H, I)) * 0.02)
    out, r = moe.layer(x, Wr, None, lambda e: one, shared, 1, H, I)
    assert np.all(r["g"] == 1.0)
    want = moe.ffn(x, *shared) + moe.ffn(x, *moe.expert_weights(*one, H, I))
    assert np.allclose(out, want, rtol=0, atol=1e-13)


def test_identical_experts_make_routing_irrelevant():
    L = _tiny()
    wl = L.wl
    x, _ = W.activations(wl)
    H, I = wl.hidden, wl.inter
    same = L.expert_bytes(5)
    rng = np.random.default_rng(5)
    o1, _ = moe.layer(x, L.router_w, None, lambda e: same, None, 2, H, I)
    o2, _ = moe.layer(x, rng.standard_normal(L.router_w.shape), None, lambda e: same, None, 2, H, I)
    assert np.allclose(o1, o2, rtol=0, atol=1e-13)


def _scale_down(raw_down):
    d = raw_down.copy()
    for lo in (80, 82):
        v = d[:, lo:lo + 2].copy().view("<f2").astype(np.float32) * 2
        d[:, lo:lo + 2] = v.astype(np.float16).view(np.uint8).reshape(-1, 2)
    return d


def test_doubling_down_scales_doubles_output_exactly():
    L = _tiny()
    wl = L.wl
    x, _ = W.activations(wl)
    H, I = wl.hidden, wl.inter
    o1, _ = moe.layer(x, L.router_w, None, L.expert_bytes, None, wl.topk, H, I)
    dbl = lambda e: (L.expert_bytes(e)[0], L.expert_bytes(e)[1], _scale_down(L.expert_bytes(e)[2]))
    o2, _ = moe.layer(x, L.router_w, None, dbl, None, wl.topk, H, I)
    assert np.array_equal(o2, 2 * o1)


# ----------------------------------------------------------------- RMSNorm / stack
def test_rmsnorm_closed_forms():
    h = np.array([[1.0, -1.0] * 128, [3.0] * 256, [0.0] * 255 + [16.0]])
    x = moe.rmsnorm_bf16(h, 1e-6)
    assert np.array_equal(x[0], np.sign(h[0]))                    # 1/sqrt(1+1e-6) -> bf16 1.0
    assert np.array_equal(x[1], np.ones(256))
    assert x[2, -1] == 16.0 and np.all(x[2, :-1] == 0)            # sqrt(1 + 1e-6) * ... -> 16
    tiny = moe.rmsnorm_bf16(np.zeros((1, 4)), 1e-6)
    assert np.all(tiny == 0)


def test_round_bf16_known_values():
    v = np.array([1.0, 1 + 2**-8, 1 + 3 * 2**-8, 1 + 2**-8 + 2**-40, -(1 + 2**-8), 2.0**-130 * 1.75])
    want = np.array([1.0, 1.0, 1 + 2**-6, 1 + 2**-7, -1.0, 2.0**-130 * 1.75])
    assert np.array_equal(moe._round_bf16(v), want)


def test_stack_with_zero_down_is_identity_and_one_layer_matches():
    L = _tiny()
    wl = L.wl
    H, I = wl.hidden, wl.inter
    rng = np.random.default_rng(6)
    h0 = rng.standard_normal((3, H))
    zero = lambda e: (L.expert_bytes(e)[0], L.expert_bytes(e)[1],
                      np.zeros_like(L.expert_bytes(e)[2]))
    layer0 = dict(router_w=L.router_w, router_b=None, expert_bytes=zero, shared=None)
    h, _ = moe.stack(h0, [layer0, layer0], wl.topk, H, I, 1e-6)
    assert np.array_equal(h, h0)
    layer1 = L.oracle_layer()
    h, _ = moe.stack(h0, [layer1], wl.topk, H, I, 1e-6)
    want = h0 + moe.layer(moe.rmsnorm_bf16(h0, 1e-6), L.router_w, None, L.expert_bytes,
                          None, wl.topk, H, I)[0]
    assert np.array_equal(h, want)


# ----------------------------------------------------------------- stack composition, closed form
def _onehot_signed_q2(rows, cols, entries):
    """Q2 bytes [rows * cols/256, 84] of a matrix whose row r holds at most one nonzero
    W[r, c] = v, entries = {r: (c, v)}.  A positive v is d * sc * q with sc = q = 1,
    d = v (fp16-exact) and no min; a negative v uses the subtracted min: m_j = 1,
    dmin = -v, and every other weight of the group gets q = 1 with d * sc = -v, so
    it decodes to 0 and the chosen one (q = 0) to v."""
    raw = np.zeros((rows, cols // 256, 84), dtype=np.uint8)
    for r, (c, v) in entries.items():
        blk = raw[r, c // 256]
        i = c % 256
        j = i // 16
        mag = np.float16(abs(v))
        assert float(mag) == abs(v)
        if v > 0:
            blk[j] = 1                                    # sc_j = 1, m_j = 0
            blk[16 + i // 4] |= 1 << (2 * (i % 4))        # q_i = 1
            blk[80:82] = np.frombuffer(mag.tobytes(), dtype=np.uint8)
        else:
            blk[j] = 1 | (1 << 4)                         # sc_j = 1, m_j = 1
            for ii in range(16 * j, 16 * j + 16):
                if ii != i:
                    blk[16 + ii // 4] |= 1 << (2 * (ii % 4))
            blk[80:82] = np.frombuffer(mag.tobytes(), dtype=np.uint8)
            blk[82:84] = np.frombuffer(mag.tobytes(), dtype=np.uint8)
    return raw.reshape(-1, 84)


def test_stack_composition_closed_form():
    """Two layers, E = 2, K = 1, H = 256, I = 512, worked by hand.

    h_0 rows are +-4 (constant magnitude, so RMSNorm gives exactly the signs in
    bf16).  The router reads coordinate 0 of the layer input: logits (x_0, -x_0), so
    expert 0 is chosen when x_0 = +1 and expert 1 when x_0 = -1, with gate 1.
    Gate rows read x_0 times +-64 so that silu sees +64 and returns exactly 64
    (e^-64 vanishes next to 1 in fp64); up row j reads x_j times s_u, down row k
    reads h_k times s_d for k in a chosen set, else 0.  So an expert adds
    s_d * 64 * s_u * x_k to coordinate k of the residual stream:
      layer 1, expert 0: s_u = 1/8, s_d = -1 on F1 = {0, 3, 7, 100, 200} -> -8 x_k,
        which flips the sign of h on F1 (4 - 8 = -4) and keeps |h| = 4;
      layer 1, expert 1: down all zero;
      layer 2, expert 1: gate -64, s_u = 1/4, s_d = 1/2 on F2 = {1, 5, 100, 255} -> +8 x_k;
      layer 2, expert 0: s_u = 1/8, s_d = 1 on every k -> +8 x_k.
    Token A (x_0 = +1): layer 1 takes expert 0 and flips coordinate 0, so layer 2 sees
    x_0 = -1 and takes expert 1: h_2 = s' (4 + 8 [k in F2]), s' = s with F1 flipped.
    Token B (x_0 = -1): layer 1 takes expert 1 (no change), layer 2 expert 1 again:
    h_2 = s (4 + 8 [k in F2]).
    Each stage is exact in fp64, so the comparison is exact.  This fails if the
    router or the experts read h instead of RMSNorm(h) (inputs of +-4: a 16x larger
    expert output), if the residual add is dropped or applied to the normalised input,
    or if RMSNorm is taken once from h_0 (layer 2 would pick expert 0 for token A)."""
    H, I = 256, 512
    rng = np.random.default_rng(11)
    F1, F2 = [0, 3, 7, 100, 200], [1, 5, 100, 255]
    zero_lo = np.zeros((H * I // 256, 84), np.uint8)

    def expert(gate_v, s_u, down):
        g = _onehot_signed_q2(I, H, {j: (0, gate_v) for j in range(I)})
        u = _onehot_signed_q2(I, H, {j: (j, s_u) for j in range(H)})
        d = _onehot_signed_q2(H, I, down) if down else zero_lo
        return (g, u, d)

    l1 = {0: expert(64.0, 0.125, {k: (k, -1.0) for k in F1}), 1: expert(-64.0, 0.125, {})}
    l2 = {0: expert(64.0, 0.125, {k: (k, 1.0) for k in range(H)}),
          1: expert(-64.0, 0.25, {k: (k, 0.5) for k in F2})}
    Wr = np.zeros((2, H))
    Wr[0, 0], Wr[1, 0] = 1.0, -1.0
    layers = [dict(router_w=Wr, router_b=None, expert_bytes=l1.__getitem__, shared=None),
              dict(router_w=Wr, router_b=None, expert_bytes=l2.__getitem__, shared=None)]
    s = np.where(rng.standard_normal((3, H)) >= 0, 1.0, -1.0)
    s[0, 0], s[1, 0], s[2, 0] = 1.0, -1.0, 1.0
    h, routings = moe.stack(4.0 * s, layers, 1, H, I, 1e-6)

    f2 = np.zeros(H)
    f2[F2] = 1.0
    want = np.empty_like(s)
    for t in range(3):
        sp = s[t].copy()
        if s[t, 0] > 0:
            sp[F1] = -sp[F1]                      # layer 1, expert 0 flips F1
        want[t] = sp * (4.0 + 8.0 * f2)           # layer 2, expert 1 adds 8 x_k on F2
    assert routings[0]["idx"][:, 0].tolist() == [0, 1, 0]
    assert routings[1]["idx"][:, 0].tolist() == [1, 1, 1]
    assert np.all(routings[0]["g"] == 1.0) and np.all(routings[1]["g"] == 1.0)
    assert np.array_equal(h, want)
    # one layer alone: h_0 with the sign of F1 flipped for token 0
    h1, _ = moe.stack(4.0 * s[:1], layers[:1], 1, H, I, 1e-6)
    w1 = 4.0 * s[0].copy()
    w1[F1] = -w1[F1]
    assert np.array_equal(h1[0], w1)

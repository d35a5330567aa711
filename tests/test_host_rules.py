"""Arithmetic rules the kernels rely on, checked on the host.

The matrix-core router splits each fp32 weight into three bf16 terms by truncation
(hi = top 8 significant bits, mid = top 8 of the exact remainder, lo = the rest):
for |w| >= 2^-102 (the rest then stays a normal number) the rest fits a bf16 value
and hi + mid + lo equals the weight exactly, so every product with a bf16
activation is exact in fp32; below that, what is lost is under 2^-126."""
import numpy as np


def _trunc_bf16(v):
    return (v.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)


def test_truncation_split_is_exact():
    rng = np.random.default_rng(7)
    n = 1 << 20
    w = (rng.standard_normal(n) * rng.choice([1e-6, 1e-3, 0.02, 1.0, 300.0], n)).astype(np.float32)
    edge = np.array([1.0000001, -1.0000001, 3.4028235e38, -3.4028235e38, 5e-30, -7.777777e-5, 0.0, -0.0,
                     2.0 ** -100, -(2.0 ** -102) * 1.9999999], dtype=np.float32)
    w = np.concatenate([w, edge])
    hi = _trunc_bf16(w)
    r1 = (w - hi).astype(np.float32)
    mid = _trunc_bf16(r1)
    r2 = (r1 - mid).astype(np.float32)
    lo = _trunc_bf16(r2)
    assert np.array_equal(lo, r2)                                  # the rest is a bf16 value
    assert np.array_equal(hi.astype(np.float64) + mid + lo, w.astype(np.float64))
    # each product with a bf16 activation is exact in fp32
    a = _trunc_bf16(rng.standard_normal(w.size).astype(np.float32))
    for part in (hi, mid, lo):
        assert np.array_equal((part * a).astype(np.float64), part.astype(np.float64) * a)
    # tiny weights: the part a subnormal rest loses is below 2^-126
    tiny = np.array([1.1754944e-38 * 3, -2.0 ** -110 * 1.2345678, 2.0 ** -120], dtype=np.float32)
    h = _trunc_bf16(tiny)
    r = (tiny - h).astype(np.float32)
    m = _trunc_bf16(r)
    lo = _trunc_bf16((r - m).astype(np.float32))
    assert np.all(np.abs(h.astype(np.float64) + m + lo - tiny.astype(np.float64)) < 2.0 ** -126)

"""Pins of the oracle's Q8 activation mode (moe.q8_rows and ffn(act="q8")) against
hand-computed values and its stated invariants (no GPU)."""
import math

import numpy as np

from oracle import moe


def test_q8_known_values():
    # max 1.0: frexp exponent 1, s = 2^-6
    v = np.array([[1.0, -0.5, 0.25, 0.3, 2.5 / 64, 3.5 / 64]])
    assert moe.q8_rows(v).tolist() == [[1.0, -0.5, 0.25, 19 / 64, 2 / 64, 4 / 64]]   # ties to even
    # max 0.999: exponent 0, s = 2^-7, 127.87 rounds to 128 and is clamped to 127
    assert moe.q8_rows(np.array([[0.999, 0.5]])).tolist() == [[127 / 128, 64 / 128]]
    # a negative maximum: |-3| -> exponent 2, s = 2^-5
    assert moe.q8_rows(np.array([[-3.0, 1.0, 0.01]])).tolist() == [[-3.0, 1.0, 0.0]]
    assert moe.q8_rows(np.zeros((1, 8))).tolist() == [[0.0] * 8]


def test_q8_invariants_random_rows():
    rng = np.random.default_rng(0)
    v = rng.standard_normal((64, 512)) * np.exp(rng.uniform(-20, 20, (64, 1)))
    q = moe.q8_rows(v)
    amax = np.abs(v).max(axis=1, keepdims=True)
    _, e = np.frexp(amax)
    s = np.ldexp(1.0, e - 7)
    a = q / s
    assert np.all(a == np.rint(a)) and np.all(np.abs(a) <= 127)
    assert np.all(np.abs(a).max(axis=1) >= 64)                 # the scale uses the top bit
    clamped = np.abs(v / s) > 127
    assert np.all(np.abs(v - q)[~clamped] <= s.repeat(512, axis=1)[~clamped] / 2)
    assert np.all(np.abs(v - q)[clamped] <= s.repeat(512, axis=1)[clamped])


def test_ffn_q8_closed_form():
    # gate row 0 reads 2 x_0, up row 0 reads x_1, every down row reads h_0.
    # x = (1, 0.3, 0...): Q8 gives x_1 = 19/64, so h_0 = silu(2) * 19/64 = 0.5229...,
    # whose Q8 value (exponent 0, s = 2^-7) is 67/128: y_k = 67/128 for every k.
    H, I = 256, 256
    x = np.zeros((1, H))
    x[0, 0], x[0, 1] = 1.0, 0.3
    wg = np.zeros((I, H)); wg[0, 0] = 2.0
    wu = np.zeros((I, H)); wu[0, 1] = 1.0
    wd = np.zeros((H, I)); wd[:, 0] = 1.0
    h0 = 2.0 / (1.0 + math.exp(-2.0)) * 19 / 64
    assert math.floor(h0 * 128 + 0.5) == 67
    y = moe.ffn(x, wg, wu, wd, act="q8")
    assert np.all(y == 67 / 128)
    y_exact = moe.ffn(x, wg, wu, wd)
    assert np.allclose(y_exact, 2.0 / (1.0 + math.exp(-2.0)) * 0.3, rtol=1e-15)

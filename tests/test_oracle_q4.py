"""Pins of the oracle's Q4 sibling codec (oracle.q4) against closed forms, brute
force, the stated byte layout and the quantizer's invariants (no GPU)."""
import numpy as np
import pytest

from oracle import moe, q2, q4


def _pack(sc, mn, q, d16, dmin16):
    """One block packed by hand from the layout description (independent of
    q4.encode_blocks): scale/min byte per group, element 4b + s of group j in byte
    16 + 8j + 4 (s // 2) + b (low nibble for even s), fp16 d and dmin."""
    b = bytearray(148)
    for j in range(16):
        b[j] = (int(sc[j]) & 15) | ((int(mn[j]) & 15) << 4)
    for i in range(256):
        j, r = divmod(i, 16)
        bb, s = divmod(r, 4)
        b[16 + 8 * j + 4 * (s // 2) + bb] |= (int(q[i]) & 15) << (4 * (s % 2))
    b[144:146] = np.float16(d16).tobytes() if not isinstance(d16, bytes) else d16
    b[146:148] = np.float16(dmin16).tobytes() if not isinstance(dmin16, bytes) else dmin16
    return np.frombuffer(bytes(b), dtype=np.uint8)


def test_sizes():
    assert q4.BLOCK_BYTES == 148
    assert q4.BLOCK_BYTES * 8 / q4.QK == 4.625


def test_closed_form_block():
    # d = dmin = 1, sc_j = j mod 8, m_j = 15 - j, q_i = i mod 16 (i within the group):
    # w = (j mod 8) * (i mod 16) - (15 - j)
    sc = np.arange(16) % 8
    mn = 15 - np.arange(16)
    q = np.arange(256) % 16
    w = q4.decode_blocks(_pack(sc, mn, q, 1.0, 1.0))[0]
    want = [((i // 16) % 8) * (i % 16) - (15 - i // 16) for i in range(256)]
    assert w.tolist() == want


def test_single_code_position():
    # Only code i nonzero: exactly weight i moves, by d * sc_j * q.
    sc = np.full(16, 5)
    mn = np.zeros(16, dtype=int)
    for i in [0, 1, 2, 3, 4, 5, 6, 7, 8, 13, 15, 16, 17, 63, 64, 131, 200, 255]:
        q = np.zeros(256, dtype=int)
        q[i] = 11
        w = q4.decode_blocks(_pack(sc, mn, q, 0.5, 0.25))[0]
        want = np.zeros(256)
        want[i] = 0.5 * 5 * 11
        assert np.array_equal(w, want), i


def test_reserved_scale_bit_is_ignored():
    q = np.full(256, 15)
    a = q4.decode_blocks(_pack(np.full(16, 7), np.zeros(16, int), q, 1.0, 0.0))[0]
    b = q4.decode_blocks(_pack(np.full(16, 15), np.zeros(16, int), q, 1.0, 0.0))[0]   # bit 3 set
    assert np.all(a == 105.0) and np.array_equal(a, b)


def test_min_subtracted_and_zero_scales():
    w = q4.decode_blocks(_pack(np.zeros(16, int), np.arange(16), np.full(256, 9), 1.0, 0.125))[0]
    assert np.array_equal(w, -0.125 * np.repeat(np.arange(16), 16))
    rng = np.random.default_rng(0)
    w = q4.decode_blocks(_pack(rng.integers(0, 8, 16), rng.integers(0, 16, 16), rng.integers(0, 16, 256),
                               0.0, 0.0))[0]
    assert np.all(w == 0)


def test_decode_rounds_once_and_subnormal_scales():
    sc, mn, q = np.full(16, 7), np.full(16, 1), np.full(256, 15)
    d, dmin = 2048.0, 2.0 ** -14 * 1.5
    w = q4.decode_blocks(_pack(sc, mn, q, d, dmin))[0]
    assert np.all(w == np.float32(105 * 2048.0 - dmin))
    w = q4.decode_blocks(_pack(sc, np.full(16, 15), q, (0x0010).to_bytes(2, "little"),
                               (0x0001).to_bytes(2, "little")))[0]
    assert np.all(w == np.float32(105 * 2.0 ** -20 - 15 * 2.0 ** -24))


def test_f16_cover_is_smallest():
    rng = np.random.default_rng(1)
    targets = np.concatenate([rng.random(2000).astype(np.float32) * 3,
                              (rng.random(500) * 1e-4).astype(np.float32),
                              np.float32(7) * np.array([1, 0.5, 2.0 ** -20], dtype=np.float32)])
    for steps in (7, 15):
        h = q4._f16_cover(targets, steps)
        assert np.all(steps * h.astype(np.float64) >= targets)
        below = (h.view(np.uint16) - 1).view(np.float16).astype(np.float64)
        assert np.all((h.view(np.uint16) == 0) | (steps * below < targets))


def _blocks(seed, n=512, sigma=0.02):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((n, 256)) * sigma).astype(np.float32)


def _fields(raw):
    sc = (raw[:, :16] & 7).astype(np.float64)
    d = raw[:, 144:146].copy().view("<f2").astype(np.float64)
    return sc, d


def _codes(raw):
    """Codes read back by the layout rule (not through q4._codes)."""
    q = np.empty((raw.shape[0], 256), dtype=np.int64)
    for i in range(256):
        j, r = divmod(i, 16)
        b, s = divmod(r, 4)
        q[:, i] = (raw[:, 16 + 8 * j + 4 * (s // 2) + b] >> (4 * (s % 2))) & 15
    return q


def test_quantizer_error_bound_and_fields():
    for seed, sigma in [(0, 0.02), (1, 1.0), (2, 1e-3)]:
        x = _blocks(seed, sigma=sigma)
        raw = q4.encode_blocks(x)
        w = q4.decode_blocks(raw)
        sc, d = _fields(raw)
        step = np.repeat(d * sc, 16, axis=1)
        ulp = np.spacing(np.maximum(np.abs(x), np.abs(w))).astype(np.float64)
        assert np.all(np.abs(x.astype(np.float64) - w) <= 0.5 * step + 4 * ulp)
        assert np.all(raw[:, :16] & 8 == 0)             # reserved bit clear, sc_j <= 7
    # 16 levels: much finer than the 2-bit format on the same weights
    x = _blocks(7)
    e4 = np.abs(q4.decode_blocks(q4.encode_blocks(x)) - x).mean()
    e2 = np.abs(q2.decode_blocks(q2.encode_blocks(x)) - x).mean()
    assert e4 < e2 / 3


def test_quantizer_monotone_within_group():
    x = _blocks(3)
    q = _codes(q4.encode_blocks(x))
    order = np.argsort(x.reshape(-1, 16, 16), axis=2, kind="stable")
    qs = np.take_along_axis(q.reshape(-1, 16, 16), order, axis=2)
    assert np.all(np.diff(qs, axis=2) >= 0)


def test_quantizer_edge_blocks():
    assert not q4.encode_blocks(np.zeros((1, 256), dtype=np.float32)).any()
    pos = np.abs(_blocks(4, 4)) + np.float32(0.01)
    raw = q4.encode_blocks(pos)
    assert np.all(raw[:, :16] >> 4 == 0) and np.all(raw[:, 146:148] == 0)   # no min
    neg = -np.abs(_blocks(5, 4)) - np.float32(0.01)
    assert np.all(q4.decode_blocks(q4.encode_blocks(neg)) <= 0)
    const = np.full((2, 256), -0.375, dtype=np.float32)
    w = q4.decode_blocks(q4.encode_blocks(const))
    assert np.all(np.abs(w - const) <= 1e-5)
    big = np.full((1, 256), 3.0, dtype=np.float32)
    raw = q4.encode_blocks(big)
    sc, d = _fields(raw)
    assert np.all(sc == 7) and np.all(_codes(raw) == 15)
    assert np.all(np.abs(q4.decode_blocks(raw) - 3.0) <= 0.5 * d * 7)
    with pytest.raises(ValueError):
        q4.encode_blocks(np.full((1, 256), 1e7, dtype=np.float32))


def test_expert_weights_dispatch_by_block_size():
    # one expert with gate/up in one format and down in the other decodes each matrix
    # with its own codec (the per-matrix mix)
    H, I = 256, 512
    rng = np.random.default_rng(8)
    g, u = (rng.standard_normal((I, H)) * 0.02).astype(np.float32), (rng.standard_normal((I, H)) * 0.02).astype(np.float32)
    dn = (rng.standard_normal((H, I)) * 0.02).astype(np.float32)
    raw = (q4.encode_matrix(g), q4.encode_matrix(u), q2.encode_matrix(dn))
    wg, wu, wd = moe.expert_weights(*raw, H, I)
    assert np.array_equal(wg, q4.decode_matrix(raw[0], I, H))
    assert np.array_equal(wd, q2.decode_matrix(raw[2], H, I))
    packed = q2.pack_expert(*raw, H, I)
    assert packed.size == 2 * I * H // 256 * 148 + H * I // 256 * 84
    back = q2.unpack_expert(packed, H, I, 148, 84)
    for a, b in zip(back, raw):
        assert np.array_equal(a, b)

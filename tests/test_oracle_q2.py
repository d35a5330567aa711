"""Pins of the oracle's Q2 codec against closed forms, brute force and the
quantizer's stated invariants (no GPU)."""
import numpy as np
import pytest

from oracle import q2


def _pack(sc, mn, q, d16, dmin16):
    """Pack one block by hand from the byte-order description (independent of
    q2.encode_blocks): scale/min nibbles, codes 4 per byte LSB first, fp16 d, dmin."""
    b = bytearray(84)
    for j in range(16):
        b[j] = (int(sc[j]) & 15) | ((int(mn[j]) & 15) << 4)
    for i in range(256):
        b[16 + i // 4] |= (int(q[i]) & 3) << (2 * (i % 4))
    b[80:82] = np.float16(d16).tobytes() if not isinstance(d16, bytes) else d16
    b[82:84] = np.float16(dmin16).tobytes() if not isinstance(dmin16, bytes) else dmin16
    return np.frombuffer(bytes(b), dtype=np.uint8)


def test_sizes():
    assert q2.BLOCK_BYTES == 84
    assert q2.BLOCK_BYTES * 8 / q2.QK == 2.625


def test_closed_form_block():
    # d = dmin = 1, sc_j = j, m_j = 15 - j, q_i = i mod 4:  w_i = j * (i mod 4) - (15 - j)
    sc = np.arange(16)
    mn = 15 - np.arange(16)
    q = np.arange(256) % 4
    w = q2.decode_blocks(_pack(sc, mn, q, 1.0, 1.0))[0]
    want = [(i // 16) * (i % 4) - (15 - i // 16) for i in range(256)]
    assert w.tolist() == want


def test_single_code_position():
    # Only code i nonzero: exactly weight i moves, by d * sc_j * q.
    sc = np.full(16, 3)
    mn = np.zeros(16, dtype=int)
    for i in [0, 1, 2, 3, 4, 15, 16, 17, 63, 64, 128, 200, 255]:
        q = np.zeros(256, dtype=int)
        q[i] = 2
        w = q2.decode_blocks(_pack(sc, mn, q, 0.5, 0.25))[0]
        want = np.zeros(256)
        want[i] = 0.5 * 3 * 2
        assert np.array_equal(w, want), i


def test_min_is_subtracted_per_group():
    sc = np.zeros(16, dtype=int)
    mn = np.arange(16)
    q = np.full(256, 3)
    w = q2.decode_blocks(_pack(sc, mn, q, 1.0, 0.125))[0]
    assert np.array_equal(w, -0.125 * np.repeat(np.arange(16), 16))


def test_power_of_two_and_subnormal_scales():
    sc = np.full(16, 15)
    mn = np.full(16, 15)
    q = np.full(256, 3)
    w = q2.decode_blocks(_pack(sc, mn, q, 2.0 ** -6, 2.0 ** -10))[0]
    assert np.all(w == 45 * 2.0 ** -6 - 15 * 2.0 ** -10)
    # fp16 subnormal d = 2^-20 (bit pattern 0x0010), dmin = smallest subnormal 2^-24
    w = q2.decode_blocks(_pack(sc, mn, q, (0x0010).to_bytes(2, "little"),
                               (0x0001).to_bytes(2, "little")))[0]
    assert np.all(w == np.float32(45 * 2.0 ** -20 - 15 * 2.0 ** -24))


def test_zero_scales_decode_to_zero():
    rng = np.random.default_rng(0)
    w = q2.decode_blocks(_pack(rng.integers(0, 16, 16), rng.integers(0, 16, 16),
                               rng.integers(0, 4, 256), 0.0, 0.0))[0]
    assert np.all(w == 0)


def test_decode_rounds_once_to_fp32():
    # d * sc * q - dmin * m needs more than 24 bits here; fp32 of the exact value.
    sc = np.full(16, 15)
    mn = np.full(16, 1)
    q = np.full(256, 3)
    d, dmin = 2048.0, 2.0 ** -14 * 1.5
    w = q2.decode_blocks(_pack(sc, mn, q, d, dmin))[0]
    exact = 45 * 2048.0 - dmin
    assert np.all(w == np.float32(exact))


def test_f16_up_is_smallest_fp16_cover():
    rng = np.random.default_rng(1)
    targets = np.concatenate([rng.random(2000).astype(np.float32) * 3,
                              (rng.random(500) * 1e-4).astype(np.float32),
                              np.float32(15) * np.array([1, 0.5, 2.0 ** -20], dtype=np.float32)])
    h = q2._f16_up(targets)
    hf = h.astype(np.float64)
    assert np.all(15 * hf >= targets)
    below = (h.view(np.uint16) - 1).view(np.float16).astype(np.float64)
    ok = (h.view(np.uint16) == 0) | (15 * below < targets)
    assert np.all(ok)


def _blocks(seed, n=512, sigma=0.02):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((n, 256)) * sigma).astype(np.float32)


def _fields(raw):
    sc = (raw[:, :16] & 15).astype(np.float64)
    d = raw[:, 80:82].copy().view("<f2").astype(np.float64)
    return sc, d


def test_quantizer_error_bound():
    for seed, sigma in [(0, 0.02), (1, 1.0), (2, 1e-3)]:
        x = _blocks(seed, sigma=sigma)
        raw = q2.encode_blocks(x)
        w = q2.decode_blocks(raw)
        sc, d = _fields(raw)
        step = np.repeat(d * sc, 16, axis=1)
        ulp = np.spacing(np.maximum(np.abs(x), np.abs(w))).astype(np.float64)
        assert np.all(np.abs(x.astype(np.float64) - w) <= 0.5 * step + 4 * ulp)


def test_quantizer_monotone_within_group():
    x = _blocks(3)
    raw = q2.encode_blocks(x)
    q = np.empty((x.shape[0], 256), dtype=np.int64)
    for s in range(4):
        q[:, s::4] = (raw[:, 16:80] >> (2 * s)) & 3
    xg = x.reshape(-1, 16, 16)
    qg = q.reshape(-1, 16, 16)
    order = np.argsort(xg, axis=2, kind="stable")
    qs = np.take_along_axis(qg, order, axis=2)
    assert np.all(np.diff(qs, axis=2) >= 0)


def test_quantizer_edge_blocks():
    zero = np.zeros((1, 256), dtype=np.float32)
    raw = q2.encode_blocks(zero)
    assert not raw.any()
    pos = np.abs(_blocks(4, 4)) + np.float32(0.01)
    raw = q2.encode_blocks(pos)
    assert np.all(raw[:, :16] >> 4 == 0)              # no min needed
    assert np.all(raw[:, 82:84] == 0)                   # dmin = 0
    neg = -np.abs(_blocks(5, 4)) - np.float32(0.01)
    w = q2.decode_blocks(q2.encode_blocks(neg))
    assert np.all(w <= 0)
    const = np.full((2, 256), -0.375, dtype=np.float32)
    raw = q2.encode_blocks(const)
    w = q2.decode_blocks(raw)
    sc, d = _fields(raw)
    assert np.all(np.abs(w - const) <= 0.5 * np.repeat(d * sc, 16, axis=1) + 1e-7)
    assert np.all(np.abs(w - const) <= 1e-5)
    big = np.full((1, 256), 3.0, dtype=np.float32)
    raw = q2.encode_blocks(big)
    w = q2.decode_blocks(raw)
    sc, d = _fields(raw)
    assert np.all(sc == 15) and np.all(np.abs(w - 3.0) <= 0.5 * d * 15)


def test_quantizer_codes_and_nibbles_in_range():
    x = _blocks(6, sigma=0.3)
    raw = q2.encode_blocks(x)
    x64 = x.reshape(-1, 16, 16).astype(np.float64)
    lo = np.minimum(0, x64.min(axis=2))
    dmin = raw[:, 82:84].copy().view("<f2").astype(np.float64)
    m = (raw[:, :16] >> 4).astype(np.float64)
    # the min reaches every weight of the group (up to one fp32 rounding)
    assert np.all(dmin * m >= -lo * (1 - 1e-6))


def test_overflowing_block_is_rejected():
    with pytest.raises(ValueError):
        q2.encode_blocks(np.full((1, 256), 1e7, dtype=np.float32))


def test_pack_expert_positions_and_roundtrip():
    H, I = 512, 256        # 2 blocks per gate/up row, 1 per down row
    rng = np.random.default_rng(7)
    g = rng.integers(0, 256, (I * 2, 84), dtype=np.uint8)
    u = rng.integers(0, 256, (I * 2, 84), dtype=np.uint8)
    d = rng.integers(0, 256, (H * 1, 84), dtype=np.uint8)
    packed = q2.pack_expert(g, u, d, H, I)
    assert packed.size == (g.size + u.size + d.size)
    blk = lambda i: packed[84 * i: 84 * (i + 1)]
    # gate row r, block b -> tile r // 32, column b, slot r % 32
    for r, b in [(0, 0), (31, 1), (32, 0), (255, 1)]:
        t, slot = r // 32, r % 32
        assert np.array_equal(blk((t * 2 + b) * 64 + slot), g[r * 2 + b])
        assert np.array_equal(blk((t * 2 + b) * 64 + 32 + slot), u[r * 2 + b])
    off = 2 * I * 2          # blocks of the gate/up part
    for r in [0, 63, 64, 511]:
        assert np.array_equal(blk(off + (r // 64) * 64 + r % 64), d[r])
    g2, u2, d2 = q2.unpack_expert(packed, H, I)
    assert np.array_equal(g2, g) and np.array_equal(u2, u) and np.array_equal(d2, d)

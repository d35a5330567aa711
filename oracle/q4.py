"""Q4 sibling super-block codec, oracle side (plain NumPy).

TEST INFRASTRUCTURE: only tests/, the smoke check and the benchmark's CPU
baseline may import this package.  It shares no code with the HIP library.

The pages ship routed experts at more than one precision: the default file is q2
with the last expert layers at q4, and the GLM layout takes routed gate/up and
down matrices at different K-quant precisions (ds4 README mirror, section "Model
Weights").  They print no layout for the 4-bit member either; this module fixes
one, the 2-bit block's geometry with 4-bit codes (148 bytes, 256 weights,
4.625 bits per weight):

    bytes   0..15   group j: bits 0..2 = scale sc_j (0..7; bit 3 reserved, ignored),
                    high nibble = min m_j
    bytes  16..143  4-bit codes; group j in bytes 16 + 8j .. 16 + 8j + 7: element
                    i = 4b + s of the group (b, s in 0..3) in byte 16 + 8j + 4 (s // 2)
                    + b, low nibble for even s, high nibble for odd s
    bytes 144..145  d     (IEEE fp16, little endian)
    bytes 146..147  dmin  (IEEE fp16, little endian)

Decoded weight i of group j:  w_i = d * sc_j * q_i - dmin * m_j,  q_i in 0..15.
The group scale has 3 bits so that every code times its scale (at most 105) stays
within a signed byte.
"""
import numpy as np

QK = 256
GROUP = 16
NGROUPS = QK // GROUP
BLOCK_BYTES = 148

assert BLOCK_BYTES * 8 / QK == 4.625


def _codes(raw):
    """q [n, 256] (uint8) from the code bytes of blocks [n, 148]."""
    n = raw.shape[0]
    cb = raw[:, 16:144].reshape(n, NGROUPS, 2, 4)     # [n, j, s // 2, b]
    q = np.empty((n, NGROUPS, 4, 4), dtype=np.uint8)   # [n, j, b, s]
    for s in range(4):
        byte = cb[:, :, s // 2, :]
        q[:, :, :, s] = (byte >> 4) if s % 2 else (byte & 0x0F)
    return q.reshape(n, QK)


def decode_blocks(raw):
    """Bytes [n, 148] (uint8) -> weights [n, 256] float32, each evaluated exactly in
    fp64 (d*sc*q and dmin*m are both exact there) and rounded once to fp32."""
    raw = np.ascontiguousarray(raw, dtype=np.uint8).reshape(-1, BLOCK_BYTES)
    sc = (raw[:, :NGROUPS] & 0x07).astype(np.float64)
    mn = (raw[:, :NGROUPS] >> 4).astype(np.float64)
    q = _codes(raw).astype(np.float64)
    d = raw[:, 144:146].copy().view("<f2").astype(np.float64)
    dmin = raw[:, 146:148].copy().view("<f2").astype(np.float64)
    w = d * np.repeat(sc, GROUP, axis=1) * q - dmin * np.repeat(mn, GROUP, axis=1)
    return w.astype(np.float32)


def decode_matrix(raw, rows, cols):
    """Row-major matrix [rows, cols] stored as rows * cols/256 blocks along each row."""
    assert cols % QK == 0
    return decode_blocks(raw).reshape(rows, cols)


def _f16_cover(target, steps):
    """Smallest fp16 value h with steps * h >= target (target >= 0, fp32): the fp16
    nearest to fp32(target / steps), one fp16 ulp up when steps * h (exact in fp32)
    falls short of the target."""
    target = np.asarray(target, dtype=np.float32)
    with np.errstate(over="ignore"):
        h = np.divide(target, np.float32(steps), dtype=np.float32).astype(np.float16)
    short = h.astype(np.float32) * np.float32(steps) < target
    hb = h.view(np.uint16).copy()
    hb[short] += 1
    h = hb.view(np.float16)
    if not np.all(np.isfinite(h)):
        raise ValueError("block range exceeds the fp16 super-scale")
    return h


def encode_blocks(w):
    """Quantize fp32 weights [n, 256] to Q4 bytes [n, 148] (coverage round-to-nearest).

    IEEE fp32, one rounding per operation, in this order:
      1. per group j: lo_j = min(0, min_i x_i), hi_j = max_i x_i
      2. dmin = smallest fp16 >= max_j(0 - lo_j) / 15;  m_j = ceil((0 - lo_j) / dmin)
         (0 when dmin = 0), at most 15;  o_j = dmin * m_j  (exact)
      3. s_j = (hi_j + o_j) / 15                (15 code steps)
      4. d = smallest fp16 >= max_j s_j / 7;  sc_j = ceil(s_j / d) (0 when d = 0), at most 7
      5. q_i = clamp(rint_even((x_i + o_j) / (d * sc_j)), 0, 15)  (0 when sc_j = 0)
    The min reaches down to every weight of the group and the 16 levels span up to
    its maximum, so |x_i - w_i| <= d*sc_j/2 up to fp32 rounding."""
    x = np.ascontiguousarray(w, dtype=np.float32).reshape(-1, NGROUPS, GROUP)
    n = x.shape[0]
    f0 = np.float32(0.0)
    lo = np.minimum(f0, x.min(axis=2))
    hi = x.max(axis=2)
    neg_lo = f0 - lo
    dmin16 = _f16_cover(neg_lo.max(axis=1), 15)
    dmin = dmin16.astype(np.float32)[:, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        m = np.where(dmin > f0, np.ceil(np.divide(neg_lo, dmin, dtype=np.float32)), f0)
    m = np.minimum(m, np.float32(15.0))
    o = dmin * m
    s = np.divide(hi + o, np.float32(15.0), dtype=np.float32)
    d16 = _f16_cover(s.max(axis=1), 7)
    d = d16.astype(np.float32)[:, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        sc = np.where(d > f0, np.ceil(np.divide(s, d, dtype=np.float32)), f0)
    sc = np.minimum(sc, np.float32(7.0))
    step = (d * sc)[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        qf = np.rint(np.divide(x + o[:, :, None], step, dtype=np.float32))
    qf = np.where(step > f0, np.clip(qf, 0, 15), 0)
    q = qf.astype(np.uint8).reshape(n, NGROUPS, 4, 4)     # [n, j, b, s]

    out = np.zeros((n, BLOCK_BYTES), dtype=np.uint8)
    out[:, :NGROUPS] = sc.astype(np.uint8) | (m.astype(np.uint8) << 4)
    cb = np.zeros((n, NGROUPS, 2, 4), dtype=np.uint8)      # [n, j, s // 2, b]
    cb[:, :, 0, :] = q[:, :, :, 0] | (q[:, :, :, 1] << 4)
    cb[:, :, 1, :] = q[:, :, :, 2] | (q[:, :, :, 3] << 4)
    out[:, 16:144] = cb.reshape(n, 128)
    out[:, 144:146] = d16.reshape(n, 1).view(np.uint8).reshape(n, 2)
    out[:, 146:148] = dmin16.reshape(n, 1).view(np.uint8).reshape(n, 2)
    return out


def encode_matrix(w):
    """fp32 matrix [rows, cols] -> Q4 bytes [rows * cols / 256, 148], row-major."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    assert w.shape[-1] % QK == 0
    return encode_blocks(w.reshape(-1, QK))

"""Q2 super-block codec, oracle side (plain NumPy).

TEST INFRASTRUCTURE: only tests/, the smoke check and the benchmark's CPU
baseline may import this package.  It shares no code with the HIP library.

Format (ds4 README mirror, section "Model Weights": routed experts stored as
2-bit, asymmetric super-block quants; the block geometry is 256 weights in 16
groups of 16, a 4-bit scale and a 4-bit min per group, fp16 d and dmin, 2.625
bits per weight).  The pages name the format but print no byte order; this
module fixes one (84 bytes per block):

    bytes  0..15  group j: low nibble = scale sc_j, high nibble = min m_j
    bytes 16..79  2-bit codes: weight i sits in byte 16 + i // 4 at bit 2*(i % 4),
                  so code dword j holds exactly group j
    bytes 80..81  d     (IEEE fp16, little endian)
    bytes 82..83  dmin  (IEEE fp16, little endian)

Decoded weight i of group j:  w_i = d * sc_j * q_i - dmin * m_j
(the min is a non-negative magnitude that is subtracted: "asymmetric").
"""
import numpy as np

QK = 256            # weights per super-block
GROUP = 16          # weights per group
NGROUPS = QK // GROUP
BLOCK_BYTES = 84

assert BLOCK_BYTES * 8 / QK == 2.625


def decode_blocks(raw):
    """Bytes [n, 84] (uint8) -> weights [n, 256] float32.

    Each weight is evaluated exactly in fp64 (d*sc*q and dmin*m are both exact
    there) and rounded once to fp32."""
    raw = np.ascontiguousarray(raw, dtype=np.uint8).reshape(-1, BLOCK_BYTES)
    n = raw.shape[0]
    sc = (raw[:, :NGROUPS] & 0x0F).astype(np.float64)
    mn = (raw[:, :NGROUPS] >> 4).astype(np.float64)
    qs = raw[:, 16:80]
    q = np.empty((n, QK), dtype=np.float64)
    for s in range(4):
        q[:, s::4] = (qs >> (2 * s)) & 3
    d = raw[:, 80:82].copy().view("<f2").astype(np.float64)        # [n, 1]
    dmin = raw[:, 82:84].copy().view("<f2").astype(np.float64)     # [n, 1]
    sc_w = np.repeat(sc, GROUP, axis=1)
    mn_w = np.repeat(mn, GROUP, axis=1)
    w = d * sc_w * q - dmin * mn_w
    return w.astype(np.float32)


def decode_matrix(raw, rows, cols):
    """Row-major matrix [rows, cols] stored as rows * cols/256 blocks along each
    row (blocks run along the reduction dimension)."""
    assert cols % QK == 0
    return decode_blocks(raw).reshape(rows, cols)


def _f16_up(target):
    """Smallest fp16 value h with 15 * h >= target (target >= 0, fp32).

    Candidate: the fp16 nearest (ties to even) to fp32(target / 15); stepped one
    fp16 ulp up when 15 * candidate (exact in fp32) falls short of target."""
    target = np.asarray(target, dtype=np.float32)
    with np.errstate(over="ignore"):
        h = np.divide(target, np.float32(15.0), dtype=np.float32).astype(np.float16)
    short = h.astype(np.float32) * np.float32(15.0) < target
    hb = h.view(np.uint16).copy()
    hb[short] += 1
    h = hb.view(np.float16)
    if not np.all(np.isfinite(h)):
        raise ValueError("block range exceeds the fp16 super-scale")
    return h


def encode_blocks(w):
    """Quantize fp32 weights [n, 256] to Q2 bytes [n, 84] (coverage round-to-nearest).

    All arithmetic is IEEE fp32, one rounding per operation, in this order:
      1. per group j: lo_j = min(0, min_i x_i), hi_j = max_i x_i
      2. dmin = smallest fp16 >= max_j(0 - lo_j) / 15;  m_j = ceil((0 - lo_j) / dmin)
         (0 when dmin = 0);  o_j = dmin * m_j  (exact)
      3. s_j = (hi_j + o_j) / 3
      4. d = smallest fp16 >= max_j s_j / 15;  sc_j = ceil(s_j / d) (0 when d = 0)
      5. q_i = clamp(rint_even((x_i + o_j) / (d * sc_j)), 0, 3)  (0 when sc_j = 0)
    The min o_j reaches down to every weight of the group and the 4 code levels
    span up to its maximum, so |x_i - w_i| <= d*sc_j/2 up to fp32 rounding."""
    x = np.ascontiguousarray(w, dtype=np.float32).reshape(-1, NGROUPS, GROUP)
    n = x.shape[0]
    f0 = np.float32(0.0)
    lo = np.minimum(f0, x.min(axis=2))                      # [n, 16]
    hi = x.max(axis=2)
    neg_lo = f0 - lo                                        # +0 for an empty min
    dmin16 = _f16_up(neg_lo.max(axis=1))                    # [n]
    dmin = dmin16.astype(np.float32)[:, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        m = np.where(dmin > f0, np.ceil(np.divide(neg_lo, dmin, dtype=np.float32)), f0)
    m = np.minimum(m, np.float32(15.0))
    o = dmin * m                                            # exact
    s = np.divide(hi + o, np.float32(3.0), dtype=np.float32)
    d16 = _f16_up(s.max(axis=1))
    d = d16.astype(np.float32)[:, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        sc = np.where(d > f0, np.ceil(np.divide(s, d, dtype=np.float32)), f0)
    sc = np.minimum(sc, np.float32(15.0))
    step = (d * sc)[:, :, None]                             # exact
    with np.errstate(divide="ignore", invalid="ignore"):
        qf = np.rint(np.divide(x + o[:, :, None], step, dtype=np.float32))
    qf = np.where(step > f0, np.clip(qf, 0, 3), 0)
    q = qf.astype(np.uint8).reshape(n, QK)

    out = np.zeros((n, BLOCK_BYTES), dtype=np.uint8)
    out[:, :NGROUPS] = sc.astype(np.uint8) | (m.astype(np.uint8) << 4)
    out[:, 16:80] = (q[:, 0::4] | (q[:, 1::4] << 2) | (q[:, 2::4] << 4) | (q[:, 3::4] << 6))
    out[:, 80:82] = d16.reshape(n, 1).view(np.uint8).reshape(n, 2)
    out[:, 82:84] = dmin16.reshape(n, 1).view(np.uint8).reshape(n, 2)
    return out


def encode_matrix(w):
    """fp32 matrix [rows, cols] -> Q2 bytes [rows * cols / 256, 84], row-major."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    assert w.shape[-1] % QK == 0
    return encode_blocks(w.reshape(-1, QK))


# ------------------------------------------------------------------ expert layout
# A routed expert is stored as row tiles so that any run of consecutive block
# columns of 64 rows is one contiguous span of bytes:
#   gate/up: I/32 tiles; tile t holds block column b = 0..H/256-1 of 64 rows,
#            slots 0..31 = gate rows 32t..32t+31, slots 32..63 = up rows 32t..32t+31
#            (byte order [t][b][slot][84]);
#   down:    H/64 tiles; tile t holds block column b = 0..I/256-1 of down rows
#            64t..64t+63 ([t][b][slot][84]).
# The expert is the gate/up tiles followed by the down tiles.


def pack_expert(gate, up, down, hidden, inter):
    """Row-major block bytes of gate [I rows x H/256], up [I x H/256], down [H x I/256]
    (each [n_blocks, block bytes]: 84 for this module's blocks, 148 for the Q4
    sibling of oracle.q4) -> the expert's tiled bytes (1-D uint8)."""
    nbh, nbi = hidden // QK, inter // QK
    gate, up, down = (np.asarray(a, np.uint8) for a in (gate, up, down))
    bg, bd = gate.shape[-1], down.shape[-1]
    assert up.shape[-1] == bg
    g = gate.reshape(inter // 32, 32, nbh, bg)
    u = up.reshape(inter // 32, 32, nbh, bg)
    gu = np.concatenate([g, u], axis=1)                  # [t, slot 64, b, bytes]
    gu = gu.transpose(0, 2, 1, 3)                         # [t, b, slot, bytes]
    d = down.reshape(hidden // 64, 64, nbi, bd).transpose(0, 2, 1, 3)
    return np.concatenate([gu.reshape(-1), d.reshape(-1)])


def unpack_expert(raw, hidden, inter, gu_bytes=BLOCK_BYTES, down_bytes=BLOCK_BYTES):
    """Inverse of pack_expert: tiled expert bytes -> row-major (gate, up, down) bytes."""
    nbh, nbi = hidden // QK, inter // QK
    raw = np.asarray(raw, np.uint8).reshape(-1)
    ngu = 2 * inter * nbh * gu_bytes
    gu = raw[:ngu].reshape(inter // 32, nbh, 64, gu_bytes).transpose(0, 2, 1, 3)
    gate = gu[:, :32].reshape(inter * nbh, gu_bytes)
    up = gu[:, 32:].reshape(inter * nbh, gu_bytes)
    d = raw[ngu:].reshape(hidden // 64, nbi, 64, down_bytes).transpose(0, 2, 1, 3)
    return gate, up, d.reshape(hidden * nbi, down_bytes)

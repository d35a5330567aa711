"""Seeded synthetic inputs (host side).

Every random tensor of a workload is a pure function of (seed, stream, index):
value i of stream s under seed k is drawn from one Philox4x32-10 call with
counter (i_lo, i_hi, s_lo, s_hi) and key (k_lo, k_hi).

Gaussian draws use no transcendental function, so that this module and the
device generator produce bit-identical fp32 values: the 128 output bits are
split into eight 16-bit integers u_0..u_7, their sum S (an Irwin-Hall sum, exact
in integers) is centred, converted to fp32 exactly, and multiplied once by an
fp32 constant c = sigma / sd(S).  The result has mean 0 and standard deviation
sigma; its tails stop at +-4.9 sigma.

bf16 tensors are the fp32 draws rounded to nearest-even.

This module holds no arithmetic of the MoE layer itself; it only makes inputs.
"""
import math

import numpy as np

from .philox import philox4x32_10

# Irwin-Hall sum of eight uniform 16-bit integers: mean 8 * 65535 / 2, variance
# 8 * (65536^2 - 1) / 12.
IH_TERMS = 8
IH_MEAN = IH_TERMS * 65535 // 2          # 262140, exact
IH_SD = math.sqrt(IH_TERMS * (65536.0 ** 2 - 1.0) / 12.0)


def normal_scale(sigma):
    """fp32 multiplier that maps a centred Irwin-Hall sum to N(0, sigma^2)."""
    return np.float32(sigma / IH_SD)


def _seed_words(seed):
    return int(seed) & 0xFFFFFFFF, (int(seed) >> 32) & 0xFFFFFFFF


def irwin_hall_centred(seed, stream, start, n):
    """Centred Irwin-Hall sums for indices start .. start+n-1 as int32."""
    idx = np.arange(start, start + n, dtype=np.uint64)
    c0 = idx & np.uint64(0xFFFFFFFF)
    c1 = idx >> np.uint64(32)
    s = int(stream)
    k0, k1 = _seed_words(seed)
    r = philox4x32_10(c0, c1, s & 0xFFFFFFFF, (s >> 32) & 0xFFFFFFFF, k0, k1)
    total = np.zeros(n, dtype=np.int64)
    for w in r:
        w = w.astype(np.int64)
        total += (w & 0xFFFF) + (w >> 16)
    return (total - IH_MEAN).astype(np.int32)


def normal_f32(seed, stream, n, sigma, start=0, chunk=1 << 22):
    """n fp32 draws of N(0, sigma^2) from (seed, stream), indices start...

    value = fp32(S - mean) * fp32(sigma / sd(S)), one IEEE fp32 multiply."""
    c = normal_scale(sigma)
    out = np.empty(n, dtype=np.float32)
    for a in range(0, n, chunk):
        b = min(n, a + chunk)
        z = irwin_hall_centred(seed, stream, start + a, b - a).astype(np.float32)
        np.multiply(z, c, out=out[a:b])
    return out


def f32_to_bf16_bits(x):
    """Round fp32 to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16_bits(seed, stream, n, sigma, start=0):
    return f32_to_bf16_bits(normal_f32(seed, stream, n, sigma, start))

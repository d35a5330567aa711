"""Seeded synthetic inputs shared by the tests, the oracle and the benchmark.

Holds only random-number generation and the workload definitions; none of the
MoE layer's arithmetic lives here.
"""
import ctypes
import os
import subprocess

import numpy as np

from . import gen
from .gen import (normal_scale, f32_to_bf16_bits, bf16_bits_to_f32)

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth_host.c")
_SO = os.path.join(_HERE, "_synth_host.so")
_lib = None


def build_host_lib():
    """Compile the C generator (gcc, OpenMP).  No fast-math: results must be
    the IEEE fp32 products the definition states."""
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-shared", "-fPIC",
           "-o", _SO + ".tmp", _SRC]
    subprocess.check_call(cmd)
    os.replace(_SO + ".tmp", _SO)


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
            build_host_lib()
        lib = ctypes.CDLL(_SO)
        lib.synth_normal_f32.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                         ctypes.c_int64, ctypes.c_float, ctypes.c_void_p]
        lib.synth_philox.argtypes = [ctypes.c_void_p] * 3
        _lib = lib
    return _lib


def philox_c(ctr, key):
    lib = _load()
    c = np.asarray(ctr, dtype=np.uint32)
    k = np.asarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib.synth_philox(c.ctypes.data, k.ctypes.data, out.ctypes.data)
    return out


def normal_f32(seed, stream, n, sigma, start=0):
    """n fp32 N(0, sigma^2) draws of (seed, stream) from index `start` (C path)."""
    out = np.empty(int(n), dtype=np.float32)
    if n:
        _load().synth_normal_f32(int(seed), int(stream), int(start), int(n),
                                 float(normal_scale(sigma)), out.ctypes.data)
    return out


def normal_bf16_bits(seed, stream, n, sigma, start=0):
    return f32_to_bf16_bits(normal_f32(seed, stream, n, sigma, start))

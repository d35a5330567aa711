"""C ABI on the host (no GPU): the library loads, exports every function the header
declares, and rejects invalid arguments with the documented status before any HIP
call (the fake device pointers below are never dereferenced)."""
import ctypes
import os
import re

import pytest

import bit_quantized_routed_amd as mq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_q2.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mq.LIB_PATH):
        from bit_quantized_routed_amd import build
        build.build()
    return mq.library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_q2_\w+)\s*\(", text)))


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(mq.EXPORTS)


def test_constants(lib):
    assert mq.block_bytes() == 84
    s = mq.make_shape(7168, 2048, 256, 2048)
    assert mq.expert_bytes(s) == 14_450_688
    for st in (mq.OK, mq.EINVAL, mq.EUNSUPPORTED, mq.EWORKSPACE, mq.EHIP):
        assert lib.moe_q2_status_string(st)
    assert lib.moe_q2_status_string(-99) == b"unknown status"


def _ws_status(shape, T, K):
    n = ctypes.c_size_t(0)
    return mq.library().moe_q2_workspace_size(ctypes.byref(shape), T, K, ctypes.byref(n)), n.value


@pytest.mark.parametrize("kw,status", [
    (dict(hidden=7000), mq.EUNSUPPORTED), (dict(inter=2000), mq.EUNSUPPORTED),
    (dict(n_experts=0), mq.EUNSUPPORTED), (dict(n_experts=513), mq.EUNSUPPORTED),
    (dict(shared_inter=100), mq.EUNSUPPORTED), (dict(act_dtype=7), mq.EINVAL),
    (dict(flags=64), mq.EINVAL), (dict(flags=mq.PATH_DECODE | mq.PATH_PREFILL), mq.EINVAL),
])
def test_workspace_size_rejects(lib, kw, status):
    base = dict(hidden=7168, inter=2048, n_experts=256, shared_inter=2048, act_dtype=mq.BF16, flags=0)
    base.update(kw)
    s = mq.make_shape(**base)
    assert _ws_status(s, 32, 8)[0] == status


def test_workspace_size_values(lib):
    s = mq.make_shape(7168, 2048, 256, 2048)
    rc, n1 = _ws_status(s, 1, 8)
    rc2, n32 = _ws_status(s, 32, 8)
    assert rc == 0 and rc2 == 0 and 0 < n1 < n32
    assert _ws_status(s, -1, 8)[0] == mq.EINVAL
    assert _ws_status(s, 4, 0)[0] == mq.EINVAL
    assert _ws_status(s, 4, 17)[0] == mq.EINVAL


A = 1 << 20          # fake 16-byte (and 256-byte) aligned "device" addresses, never touched


def _fwd(shape, T=4, K=2, x=A, wr=2 * A, ex=3 * A, sh=None, out=8 * A, ws=16 * A, wsb=1 << 40,
         bias=None):
    lib = mq.library()
    return lib.moe_q2_forward(x, wr, ex, sh, K, out, ctypes.byref(shape), T, bias, ws, wsb, None, None)


def test_forward_validation(lib):
    s = mq.make_shape(256, 512, 8, 0, mq.F32)
    assert _fwd(s, T=0) == mq.OK                                     # no-op
    assert _fwd(s, x=None) == mq.EINVAL
    assert _fwd(s, wr=None) == mq.EINVAL
    assert _fwd(s, ex=None) == mq.EINVAL
    assert _fwd(s, out=None) == mq.EINVAL
    assert _fwd(s, T=-1) == mq.EINVAL
    assert _fwd(s, K=0) == mq.EINVAL and _fwd(s, K=9) == mq.EINVAL
    assert _fwd(s, x=A + 4) == mq.EINVAL                              # misaligned activations
    assert _fwd(s, ex=3 * A + 8) == mq.EINVAL                         # misaligned experts
    assert _fwd(s, sh=5 * A) == mq.EINVAL                             # shared given, Is = 0
    s2 = mq.make_shape(256, 512, 8, 256, mq.F32)
    assert _fwd(s2, sh=None) == mq.EINVAL                             # Is > 0, shared missing
    assert _fwd(s, ws=None) == mq.EWORKSPACE
    assert _fwd(s, wsb=100) == mq.EWORKSPACE
    assert _fwd(s, ws=16 * A + 64) == mq.EINVAL                       # workspace not 256-aligned
    assert _fwd(s, out=A) == mq.EINVAL                                # out aliases x, no flags
    s3 = mq.make_shape(256, 512, 8, 0, mq.F32, mq.PRE_RMSNORM | mq.RESIDUAL_ADD)
    n = ctypes.c_size_t(0)
    assert lib.moe_q2_workspace_size(ctypes.byref(s3), 4, 2, ctypes.byref(n)) == 0
    s4 = mq.make_shape(256, 512, 8, 0, mq.F32, mq.PRE_RMSNORM, rms_eps=-1.0)
    assert _fwd(s4) == mq.EINVAL


def test_setup_helpers_validation(lib):
    assert lib.moe_q2_quantize(None, 0, None, None) == mq.OK
    assert lib.moe_q2_quantize(A + 4, 1, 2 * A, None) == mq.EINVAL
    assert lib.moe_q2_quantize(None, 1, 2 * A, None) == mq.EINVAL
    assert lib.moe_q2_quantize(A, -1, 2 * A, None) == mq.EINVAL
    assert lib.moe_q2_synth_normal(0, 0, 0, 0, 1.0, mq.F32, None, None) == mq.OK
    assert lib.moe_q2_synth_normal(0, 0, 0, 10, 1.0, 5, A, None) == mq.EINVAL
    assert lib.moe_q2_synth_normal(0, 0, 0, 10, 1.0, mq.F32, None, None) == mq.EINVAL
    assert lib.moe_q2_pack_expert(A, A, A, 100, 256, A, None) == mq.EUNSUPPORTED
    assert lib.moe_q2_pack_expert(None, A, A, 256, 256, A, None) == mq.EINVAL

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
    assert lib.moe_q2_q4_block_bytes() == 148 == mq.Q4_BLOCK_BYTES
    s = mq.make_shape(7168, 2048, 256, 2048)
    assert mq.expert_bytes(s) == 14_450_688
    nb = 7168 * 2048 // 256
    assert mq.expert_bytes(mq.make_shape(7168, 2048, 256, 2048, flags=mq.GU_Q4)) == 2 * nb * 148 + nb * 84
    assert mq.expert_bytes(mq.make_shape(7168, 2048, 256, 2048, flags=mq.DOWN_Q4)) == 2 * nb * 84 + nb * 148
    assert mq.expert_bytes(mq.make_shape(7168, 2048, 256, 2048, flags=mq.GU_Q4 | mq.DOWN_Q4)) == 3 * nb * 148
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
    (dict(flags=1024), mq.EINVAL), (dict(flags=mq.PATH_DECODE | mq.PATH_PREFILL), mq.EINVAL),
    (dict(flags=mq.BATCH_INVARIANT | mq.PATH_PREFILL), mq.EINVAL),
    (dict(flags=mq.BATCH_INVARIANT | mq.DECODE_VALU), mq.EUNSUPPORTED),
    (dict(flags=mq.ACT_Q8 | mq.DECODE_VALU), mq.EUNSUPPORTED),
    (dict(flags=mq.GU_Q4 | mq.DECODE_VALU), mq.EUNSUPPORTED),
    (dict(flags=mq.BATCH_INVARIANT, act_dtype=mq.F32), mq.EUNSUPPORTED),   # fp32 input + shared expert
])
def test_workspace_size_rejects(lib, kw, status):
    base = dict(hidden=7168, inter=2048, n_experts=256, shared_inter=2048, act_dtype=mq.BF16, flags=0)
    base.update(kw)
    s = mq.make_shape(**base)
    assert _ws_status(s, 32, 8)[0] == status


@pytest.mark.parametrize("H,I,K,T,ok", [
    (7168, 2048, 8, 65535, True),            # the largest token count: 65535 * 8 * 2 * 2048 < 2^31
    (7168, 2048, 8, 65536, False),           # above MOE_Q2_MAX_TOKENS
    (7168, 2048, 16, 32767, True),           # (T K + 1) 2 I = 2147422208 <= INT32_MAX
    (7168, 2048, 16, 32768, False),          # (T K + 1) 2 I > INT32_MAX
    (16384, 16384, 16, 4095, True),          # (4095 * 16 + 1) * 32768 < 2^31
    (16384, 16384, 16, 4096, False),
    (16384, 256, 1, 65534, True),            # (T + 1) 2 H = 65535 * 32768 < 2^31
])
def test_token_envelope(lib, H, I, K, T, ok):
    """The token envelope: the combine's token grid and the 32-bit byte offsets of
    the activation rows (header: MOE_Q2_MAX_TOKENS and the two row-byte limits)."""
    s = mq.make_shape(H, I, 256, 0)
    rc, _ = _ws_status(s, T, K)
    assert rc == (mq.OK if ok else mq.EUNSUPPORTED)
    if ok:
        assert (T + 1) * 2 * H <= 2**31 - 1 and (T * K + 1) * 2 * I <= 2**31 - 1
    if not ok:                        # rejected before any HIP call (fake pointers never used)
        assert _fwd(s, T=T, K=K, wsb=1 << 60) == mq.EUNSUPPORTED


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
    assert lib.moe_q2_quantize(None, 0, 256, None, None) == mq.OK
    assert lib.moe_q2_quantize(None, 5, 0, None, None) == mq.OK
    assert lib.moe_q2_quantize(A + 4, 1, 256, 2 * A, None) == mq.EINVAL
    assert lib.moe_q2_quantize(None, 1, 256, 2 * A, None) == mq.EINVAL
    assert lib.moe_q2_quantize(A, -1, 256, 2 * A, None) == mq.EINVAL
    assert lib.moe_q2_quantize(A, 2, 100, 2 * A, None) == mq.EINVAL     # k not a multiple of 256
    assert lib.moe_q2_quantize(A, 1 << 62, 1024, 2 * A, None) == mq.EINVAL   # rows * k overflows
    assert lib.moe_q2_synth_normal(0, 0, 0, 0, 1.0, mq.F32, None, None) == mq.OK
    assert lib.moe_q2_synth_normal(0, 0, 0, 10, 1.0, 5, A, None) == mq.EINVAL
    assert lib.moe_q2_synth_normal(0, 0, 0, 10, 1.0, mq.F32, None, None) == mq.EINVAL
    bad = mq.make_shape(100, 256, 8, 0)
    ok = mq.make_shape(256, 256, 8, 0)
    assert lib.moe_q2_pack_expert(A, A, A, ctypes.byref(bad), A, None) == mq.EUNSUPPORTED
    assert lib.moe_q2_pack_expert(None, A, A, ctypes.byref(ok), A, None) == mq.EINVAL
    assert lib.moe_q2_pack_expert(A, A, A, None, A, None) == mq.EINVAL
    assert lib.moe_q2_quantize_q4(A + 4, 1, 256, 2 * A, None) == mq.EINVAL
    assert lib.moe_q2_quantize_q4(None, 0, 256, None, None) == mq.OK


def test_noalloc_validation(lib):
    """moe_q2_forward_noalloc validates like moe_q2_forward and refuses a batch whose
    workspace exceeds its fixed per-device array, all before any HIP call."""
    f = lib.moe_q2_forward_noalloc
    s = mq.make_shape(7168, 2048, 256, 2048)
    assert f(A, 2 * A, 3 * A, 5 * A, 8, 8 * A, ctypes.byref(s), 0, None, None, None) == mq.OK
    assert f(None, 2 * A, 3 * A, 5 * A, 8, 8 * A, ctypes.byref(s), 4, None, None, None) == mq.EINVAL
    assert f(A, 2 * A, 3 * A, None, 8, 8 * A, ctypes.byref(s), 4, None, None, None) == mq.EINVAL
    assert mq.workspace_size(s, 255, 8) > mq.NOALLOC_MAX_BYTES
    assert f(A, 2 * A, 3 * A, 5 * A, 8, 64 * A, ctypes.byref(s), 255, None, None, None) == mq.EUNSUPPORTED
    assert mq.workspace_size(s, 96, 8) <= mq.NOALLOC_MAX_BYTES      # the verification micro-batch fits


def test_plans(lib):
    """Path choices (moe_q2_describe): batch-invariant calls keep one set of splits
    (gate/up at most 2, down unsplit: fixed by the shape), the router split and the
    decode kernels at every batch size; Q4 matrices take the prefill
    kernels from the same batch size as Q2 (and when forced); Q8 activations halve the
    digit buffers."""
    s = mq.make_shape(7168, 2048, 256, 2048)
    one = mq.describe(s, 1, 8)
    bi = mq.make_shape(7168, 2048, 256, 2048, flags=mq.BATCH_INVARIANT)
    plans = [mq.describe(bi, T, 8) for T in (1, 5, 32, 96, 255, 2048)]
    assert (one["split_gate_up"], one["split_down"]) == (4, 2)
    for p in plans:
        assert p["path"] == mq.PATH_DECODE and p["routed_kernel"] == 0
        assert (p["split_gate_up"], p["split_down"]) == (2, 1)
        assert p["router_splits"] == plans[0]["router_splits"] == 16
    # the fixed gate/up splits run merged (one work-group per unit and tile group) from
    # the batch sizes whose own plan needs no split; never without the batch-invariant flag
    assert [p["merged"] for p in plans] == [0, 1, 1, 1, 1, 1]
    assert all(mq.describe(s, T, 8)["merged"] == 0 for T in (1, 5, 32, 96, 255))
    assert mq.describe(s, 2048, 8)["path"] == mq.PATH_PREFILL
    q4 = mq.make_shape(7168, 2048, 256, 2048, flags=mq.GU_Q4 | mq.DOWN_Q4)
    assert mq.describe(q4, 2048, 8)["path"] == mq.PATH_PREFILL
    assert mq.describe(q4, 32, 8)["path"] == mq.PATH_DECODE
    q4pf = mq.make_shape(7168, 2048, 256, 2048, flags=mq.DOWN_Q4 | mq.PATH_PREFILL)
    assert mq.describe(q4pf, 32, 8)["routed_kernel"] == 2
    q8 = mq.make_shape(7168, 2048, 256, 2048, flags=mq.ACT_Q8)
    assert mq.workspace_size(q8, 32, 8) < mq.workspace_size(s, 32, 8)


def test_cache_validation(lib):
    """Expert-cache entry points: state size, and the checks made before any HIP call."""
    assert mq.cache_state_bytes(128, 256) == 4 * (8 + 2 * 128 + 2 * 256)
    assert mq.cache_state_bytes(0, 256) == 0 and mq.cache_state_bytes(2049, 256) == 0
    s = mq.make_shape(7168, 2048, 256, 2048)
    eb = mq.expert_bytes(s)
    f = lib.moe_q2_forward_cached

    def call(cache, key_base=0, T=32, shape=s):
        return f(A, 2 * A, 3 * A, key_base, ctypes.byref(cache), 5 * A, 8, 8 * A, ctypes.byref(shape), T,
                 None, 16 * A, 1 << 40, None, None)
    good = mq.make_cache(64 * A, eb, 256, 256, 32 * A)
    assert call(good) == mq.EINVAL          # host_experts not pinned host memory: refused by the pointer query
    assert call(good, key_base=1) == mq.EINVAL                                         # keys beyond n_keys
    assert call(mq.make_cache(64 * A, eb - 16, 256, 256, 32 * A)) == mq.EINVAL          # slot too small
    assert call(mq.make_cache(64 * A, eb, 256, 256, None)) == mq.EINVAL                 # no state
    assert call(mq.make_cache(64 * A, eb, 0, 256, 32 * A)) == mq.EINVAL
    assert call(mq.make_cache(64 * A, eb, 256, 256, 32 * A, policy=2)) == mq.EINVAL       # unknown policy
    bad = mq.make_cache(64 * A, eb, 256, 256, 32 * A, policy=mq.CACHE_LRU_ADMIT)
    bad.reserved = 1
    assert call(bad) == mq.EINVAL
    sv = mq.make_shape(7168, 2048, 256, 2048, flags=mq.DECODE_VALU)
    assert call(good, shape=sv) == mq.EUNSUPPORTED
    assert call(good, T=0) == mq.OK                                                     # empty batch
    assert lib.moe_q2_cache_reset(None, None) == mq.EINVAL

"""Python binding of libmoe_q2 (the 2-bit routed-expert MoE layer for MI355X).

Argument marshalling only: torch tensors are passed as raw device pointers and
every step of the layer runs in the HIP library.  The library must be built
(`python -m bit_quantized_routed_amd.build` or __graft_entry__.build()); there is
no fallback path.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_q2.so")

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP = 0, -1, -2, -3, -4
F32, BF16 = 0, 1
PATH_AUTO, PATH_DECODE, PATH_PREFILL, PRE_RMSNORM, RESIDUAL_ADD, DECODE_VALU, SERIAL = 0, 1, 2, 4, 8, 16, 32
BATCH_INVARIANT, ACT_Q8, GU_Q4, DOWN_Q4 = 64, 128, 256, 512
PREFILL_MIN_TOKENS = 256
MAX_TOKENS = 65535
BLOCK_BYTES = 84
Q4_BLOCK_BYTES = 148

EXPORTS = ["moe_q2_block_bytes", "moe_q2_expert_bytes", "moe_q2_workspace_size",
           "moe_q2_describe", "moe_q2_forward", "moe_q2_forward_noalloc", "moe_q2_quantize",
           "moe_q2_quantize_q4", "moe_q2_q4_block_bytes", "moe_q2_pack_expert",
           "moe_q2_cache_state_bytes", "moe_q2_cache_reset", "moe_q2_forward_cached",
           "moe_q2_synth_normal", "moe_q2_status_string", "moe_q2_last_hip_error"]


class Shape(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("shared_inter", ctypes.c_int32),
                ("act_dtype", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("rms_eps", ctypes.c_float)]


class Cache(ctypes.Structure):
    _fields_ = [("slots", ctypes.c_void_p), ("slot_bytes", ctypes.c_int64), ("n_slots", ctypes.c_int32),
                ("n_keys", ctypes.c_int32), ("state", ctypes.c_void_p), ("policy", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


CACHE_MAX_SLOTS = 2048
CACHE_HDR = 8
CACHE_LRU, CACHE_LRU_ADMIT = 0, 1


class Plan(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("routed_kernel", ctypes.c_int32),
                ("shared_fused", ctypes.c_int32), ("side_branch", ctypes.c_int32),
                ("split_gate_up", ctypes.c_int32), ("split_down", ctypes.c_int32),
                ("router_splits", ctypes.c_int32), ("merged", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_size_t)]


class Trace(ctypes.Structure):
    _fields_ = [("topk_idx", ctypes.c_void_p), ("topk_w", ctypes.c_void_p),
                ("counts", ctypes.c_void_p), ("offsets", ctypes.c_void_p),
                ("perm", ctypes.c_void_p), ("events", ctypes.c_void_p)]


PHASES = ["rmsnorm", "router", "topk", "bucket", "prep_x", "gate_up", "prep_h", "down",
          "shared", "combine", "cache"]


class MoeQ2Error(RuntimeError):
    def __init__(self, status, what):
        lib = _lib()
        msg = lib.moe_q2_status_string(status).decode()
        if status == EHIP:
            msg += " (hipError %d)" % lib.moe_q2_last_hip_error()
        super().__init__("%s: status %d, %s" % (what, status, msg))
        self.status = status


_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libmoe_q2.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, u64, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                 ctypes.c_uint64, ctypes.c_size_t)
        lib.moe_q2_block_bytes.restype = sz
        lib.moe_q2_block_bytes.argtypes = []
        lib.moe_q2_expert_bytes.restype = sz
        lib.moe_q2_expert_bytes.argtypes = [ctypes.POINTER(Shape)]
        lib.moe_q2_workspace_size.restype = ctypes.c_int
        lib.moe_q2_workspace_size.argtypes = [ctypes.POINTER(Shape), i32, i32, ctypes.POINTER(sz)]
        lib.moe_q2_describe.restype = ctypes.c_int
        lib.moe_q2_describe.argtypes = [ctypes.POINTER(Shape), i32, i32, ctypes.POINTER(Plan)]
        lib.moe_q2_forward.restype = ctypes.c_int
        lib.moe_q2_forward.argtypes = [vp, vp, vp, vp, i32, vp, ctypes.POINTER(Shape), i32, vp,
                                       vp, sz, ctypes.POINTER(Trace), vp]
        lib.moe_q2_forward_noalloc.restype = ctypes.c_int
        lib.moe_q2_forward_noalloc.argtypes = [vp, vp, vp, vp, i32, vp, ctypes.POINTER(Shape), i32, vp,
                                               ctypes.POINTER(Trace), vp]
        lib.moe_q2_cache_state_bytes.restype = sz
        lib.moe_q2_cache_state_bytes.argtypes = [i32, i32]
        lib.moe_q2_cache_reset.restype = ctypes.c_int
        lib.moe_q2_cache_reset.argtypes = [ctypes.POINTER(Cache), vp]
        lib.moe_q2_forward_cached.restype = ctypes.c_int
        lib.moe_q2_forward_cached.argtypes = [vp, vp, vp, i32, ctypes.POINTER(Cache), vp, i32, vp,
                                              ctypes.POINTER(Shape), i32, vp, vp, sz, ctypes.POINTER(Trace), vp]
        lib.moe_q2_quantize.restype = ctypes.c_int
        lib.moe_q2_quantize.argtypes = [vp, i64, i64, vp, vp]
        lib.moe_q2_quantize_q4.restype = ctypes.c_int
        lib.moe_q2_quantize_q4.argtypes = [vp, i64, i64, vp, vp]
        lib.moe_q2_q4_block_bytes.restype = sz
        lib.moe_q2_q4_block_bytes.argtypes = []
        lib.moe_q2_pack_expert.restype = ctypes.c_int
        lib.moe_q2_pack_expert.argtypes = [vp, vp, vp, ctypes.POINTER(Shape), vp, vp]
        lib.moe_q2_synth_normal.restype = ctypes.c_int
        lib.moe_q2_synth_normal.argtypes = [u64, u64, u64, i64, ctypes.c_float, i32, vp, vp]
        lib.moe_q2_status_string.restype = ctypes.c_char_p
        lib.moe_q2_status_string.argtypes = [ctypes.c_int]
        lib.moe_q2_last_hip_error.restype = ctypes.c_int
        lib.moe_q2_last_hip_error.argtypes = []
        _LIB = lib
    return _LIB


def library():
    return _lib()


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_shape(hidden, inter, n_experts, shared_inter=0, act_dtype=BF16, flags=0, rms_eps=1e-6):
    return Shape(hidden, inter, n_experts, shared_inter, act_dtype, flags, rms_eps)


def block_bytes():
    return int(_lib().moe_q2_block_bytes())


def expert_bytes(shape):
    return int(_lib().moe_q2_expert_bytes(ctypes.byref(shape)))


def workspace_size(shape, n_tokens, topk):
    n = ctypes.c_size_t(0)
    rc = _lib().moe_q2_workspace_size(ctypes.byref(shape), n_tokens, topk, ctypes.byref(n))
    if rc:
        raise MoeQ2Error(rc, "moe_q2_workspace_size")
    return int(n.value)


def describe(shape, n_tokens, topk):
    """moe_q2_describe as a dict: path, routed kernel, fused shared expert, use of the
    internal stream, reduction splits, workspace bytes."""
    p = Plan()
    rc = _lib().moe_q2_describe(ctypes.byref(shape), n_tokens, topk, ctypes.byref(p))
    if rc:
        raise MoeQ2Error(rc, "moe_q2_describe")
    return {f: getattr(p, f) for f, _ in Plan._fields_}


def forward(x, router_w, experts_q2, shared_w, topk, out, shape, n_tokens, router_b=None,
            workspace=None, trace=None, stream=None, check=True):
    """moe_q2_forward on torch device tensors (raw pointers are passed through).

    trace: optional dict with any of topk_idx, topk_w, counts, offsets, perm tensors, and
    `events`: an EventSet whose 2 * len(PHASES) HIP events bracket the phases."""
    tr = None
    if trace:
        ev = trace.get("events")
        tr = Trace(*[_ptr(trace.get(k)) for k in ("topk_idx", "topk_w", "counts", "offsets", "perm")],
                   ev.array_ptr() if ev is not None else None)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = _lib().moe_q2_forward(_ptr(x), _ptr(router_w), _ptr(experts_q2), _ptr(shared_w), topk,
                               _ptr(out), ctypes.byref(shape), n_tokens, _ptr(router_b),
                               _ptr(workspace), ws_bytes, ctypes.byref(tr) if tr else None,
                               _stream(stream))
    if rc and check:
        raise MoeQ2Error(rc, "moe_q2_forward")
    return rc


NOALLOC_MAX_BYTES = 128 << 20


def _trace_struct(trace):
    if not trace:
        return None
    ev = trace.get("events")
    return Trace(*[_ptr(trace.get(k)) for k in ("topk_idx", "topk_w", "counts", "offsets", "perm")],
                 ev.array_ptr() if ev is not None else None)


def cache_state_bytes(n_slots, n_keys):
    return int(_lib().moe_q2_cache_state_bytes(n_slots, n_keys))


def make_cache(slots, slot_bytes, n_slots, n_keys, state, policy=CACHE_LRU):
    """moe_q2_cache over caller-owned device tensors: `slots` (n_slots * slot_bytes
    bytes) and `state` (cache_state_bytes(n_slots, n_keys) bytes, int32); policy
    CACHE_LRU or CACHE_LRU_ADMIT (frequency admission)."""
    return Cache(_ptr(slots), slot_bytes, n_slots, n_keys, _ptr(state), policy, 0)


def cache_reset(cache, stream=None):
    rc = _lib().moe_q2_cache_reset(ctypes.byref(cache), _stream(stream))
    if rc:
        raise MoeQ2Error(rc, "moe_q2_cache_reset")


def forward_cached(x, router_w, host_experts, key_base, cache, shared_w, topk, out, shape, n_tokens,
                   router_b=None, workspace=None, trace=None, stream=None, check=True):
    """moe_q2_forward_cached: the routed experts in pinned host memory (`host_experts`,
    a pinned tensor) behind the HBM expert cache `cache` (make_cache)."""
    tr = _trace_struct(trace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = _lib().moe_q2_forward_cached(_ptr(x), _ptr(router_w), _ptr(host_experts), key_base, ctypes.byref(cache),
                                      _ptr(shared_w), topk, _ptr(out), ctypes.byref(shape), n_tokens,
                                      _ptr(router_b), _ptr(workspace), ws_bytes,
                                      ctypes.byref(tr) if tr else None, _stream(stream))
    if rc and check:
        raise MoeQ2Error(rc, "moe_q2_forward_cached")
    return rc


def forward_noalloc(x, router_w, experts_q2, shared_w, topk, out, shape, n_tokens, router_b=None,
                    trace=None, stream=None, check=True):
    """moe_q2_forward_noalloc: the layer on the library's fixed per-device workspace
    (no workspace argument, nothing allocated; batches whose workspace exceeds
    NOALLOC_MAX_BYTES are refused)."""
    tr = None
    if trace:
        ev = trace.get("events")
        tr = Trace(*[_ptr(trace.get(k)) for k in ("topk_idx", "topk_w", "counts", "offsets", "perm")],
                   ev.array_ptr() if ev is not None else None)
    rc = _lib().moe_q2_forward_noalloc(_ptr(x), _ptr(router_w), _ptr(experts_q2), _ptr(shared_w), topk,
                                       _ptr(out), ctypes.byref(shape), n_tokens, _ptr(router_b),
                                       ctypes.byref(tr) if tr else None, _stream(stream))
    if rc and check:
        raise MoeQ2Error(rc, "moe_q2_forward_noalloc")
    return rc


def quantize(w, rows, k, blocks_out, stream=None):
    """moe_q2_quantize: row-major fp32 [rows, k] -> rows * k / 256 Q2 blocks."""
    rc = _lib().moe_q2_quantize(_ptr(w), rows, k, _ptr(blocks_out), _stream(stream))
    if rc:
        raise MoeQ2Error(rc, "moe_q2_quantize")


def quantize_q4(w, rows, k, blocks_out, stream=None):
    """moe_q2_quantize_q4: row-major fp32 [rows, k] -> rows * k / 256 Q4 sibling blocks."""
    rc = _lib().moe_q2_quantize_q4(_ptr(w), rows, k, _ptr(blocks_out), _stream(stream))
    if rc:
        raise MoeQ2Error(rc, "moe_q2_quantize_q4")


def pack_expert(gate, up, down, shape, out, stream=None):
    """moe_q2_pack_expert: row-major gate, up, down block matrices (formats from the
    shape's flags) -> the expert's tiled layout."""
    rc = _lib().moe_q2_pack_expert(_ptr(gate), _ptr(up), _ptr(down), ctypes.byref(shape), _ptr(out),
                                   _stream(stream))
    if rc:
        raise MoeQ2Error(rc, "moe_q2_pack_expert")


def synth_normal(seed, stream_id, start, n, scale, out, out_dtype=F32, stream=None):
    rc = _lib().moe_q2_synth_normal(seed, stream_id, start, n, float(scale), out_dtype, _ptr(out),
                                    _stream(stream))
    if rc:
        raise MoeQ2Error(rc, "moe_q2_synth_normal")


class EventSet:
    """2 * len(PHASES) hipEvent_t handles (created with the HIP runtime directly) that
    moe_q2_forward records around its phases; elapsed() returns per-phase ms."""

    def __init__(self, phases=None):
        """phases: names of the phases to bracket (default: all)."""
        hip = ctypes.CDLL("libamdhip64.so")
        hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                            ctypes.c_void_p]
        hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self._hip = hip
        n = 2 * len(PHASES)
        self._arr = (ctypes.c_void_p * n)()
        want = set(PHASES if phases is None else phases)
        for i in range(n):
            if PHASES[i // 2] not in want:
                self._arr[i] = None
                continue
            h = ctypes.c_void_p()
            rc = hip.hipEventCreate(ctypes.byref(h))
            if rc:
                raise RuntimeError("hipEventCreate failed: %d" % rc)
            self._arr[i] = h

    def array_ptr(self):
        return ctypes.cast(self._arr, ctypes.c_void_p).value

    def elapsed(self):
        """Per-phase durations in ms of the last recorded forward (synchronises)."""
        for i in range(len(self._arr)):
            if self._arr[i]:
                self._hip.hipEventSynchronize(self._arr[i])
        out = {}
        for i, name in enumerate(PHASES):
            if not self._arr[2 * i]:
                continue
            ms = ctypes.c_float()
            rc = self._hip.hipEventElapsedTime(ctypes.byref(ms), self._arr[2 * i], self._arr[2 * i + 1])
            out[name] = ms.value if rc == 0 else float("nan")
        return out

    def close(self):
        for i in range(len(self._arr)):
            if self._arr[i]:
                self._hip.hipEventDestroy(self._arr[i])
                self._arr[i] = None

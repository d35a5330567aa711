"""The budgeted HBM expert cache (moe_q2_forward_cached) on the GPU: a layer whose
routed experts live in pinned host memory gives the same bits as the layer resident
in HBM, over a sequence of micro-batches with different routing (hits, misses and
evictions), on the decode and prefill kernels, with one cache shared by two layers,
and under graph capture; after every call the device's cache state (slot contents,
stamps, key map, counters) equals the oracle's LRU simulation fed the same touched
experts."""
import numpy as np
import pytest
import torch

from oracle.cache import LRUCache
from synth import workloads as W
from tests.gpu_util import need_gpu, make_trace, trace_np

pytestmark = pytest.mark.gpu


class _Cache:
    def __init__(self, mq, n_slots, n_keys, slot_bytes, policy=0):
        self.slots = torch.empty(n_slots * slot_bytes, dtype=torch.uint8, device="cuda")
        self.state = torch.empty(mq.cache_state_bytes(n_slots, n_keys) // 4, dtype=torch.int32, device="cuda")
        self.c = mq.make_cache(self.slots, slot_bytes, n_slots, n_keys, self.state, policy=policy)
        self.n_slots, self.n_keys = n_slots, n_keys
        mq.cache_reset(self.c)

    def check(self, mq, oracle):
        st = self.state.cpu().numpy()
        H, n, nk = mq.CACHE_HDR, self.n_slots, self.n_keys
        key, stamp = st[H:H + n], st[H + n:H + 2 * n]
        key_slot, key_count = st[H + 2 * n:H + 2 * n + nk], st[H + 2 * n + nk:]
        assert st[0] == oracle.clock and st[1] == oracle.hits and st[2] == oracle.misses
        assert all(key_count[k] == oracle.count.get(k, 0) for k in range(nk))
        assert st[5] == oracle.last_uncached and st[6] == oracle.uncached
        assert key.tolist() == oracle.key and stamp.tolist() == oracle.stamp
        want = np.full(self.n_keys, -1)
        for s, k in enumerate(oracle.key):
            if k >= 0:
                want[k] = s
        assert np.array_equal(key_slot, want)


def _host_copy(dev):
    host = torch.empty(dev.numel(), dtype=torch.uint8, pin_memory=True)
    host.copy_(dev)
    torch.cuda.synchronize()
    return host


def _pair(mq, dl, x, T, cache, host, key_base=0, flags=0):
    """(resident output, cached output, touched experts) of one batch."""
    from bit_quantized_routed_amd import workload as dw
    wl = dl.wl
    shape = dl.shape(flags)
    ws = dw.workspace(shape, T, wl.topk)
    o1 = torch.zeros((T, wl.hidden), dtype=torch.float32, device="cuda")
    # (unwritten outputs would keep 9.0; under RESIDUAL_ADD both start from zero)
    o2 = torch.full((T, wl.hidden), 0.0 if flags & mq.RESIDUAL_ADD else 9.0, dtype=torch.float32, device="cuda")
    tr = make_trace(T, wl.topk, wl.n_experts)
    mq.forward(x, dl.router_w, dl.experts, dl.shared_w, wl.topk, o1, shape, T, router_b=dl.router_b,
               workspace=ws)
    mq.forward_cached(x, dl.router_w, host, key_base, cache.c, dl.shared_w, wl.topk, o2, shape, T,
                      router_b=dl.router_b, workspace=ws, trace=tr)
    torch.cuda.synchronize()
    touched = np.nonzero(trace_np(tr)["counts"] > 0)[0]
    return o1.cpu().numpy(), o2.cpu().numpy(), touched


@pytest.mark.parametrize("policy", [0, 1], ids=["lru", "lru_admit"])
def test_cache_decode_sequence_matches_resident_and_lru(policy):
    mq = need_gpu()
    from bit_quantized_routed_amd import workload as dw
    wl = W.WORKLOADS["decode32_zipf"]
    dl = dw.DeviceLayer(wl)
    host = _host_copy(dl.experts)
    T, E = wl.tokens, wl.n_experts
    cache = _Cache(mq, 128, E, wl.expert_bytes, policy=policy)   # half the layer's experts
    oracle = LRUCache(128, admit=policy == 1)
    xs = dw.activations(wl, tokens=4 * T)
    order = [0, 1, 2, 0, 3, 1, 1]                          # new batches, repeats (hits)
    for n, b in enumerate(order):
        x = xs[b * T:(b + 1) * T].contiguous()
        o1, o2, touched = _pair(mq, dl, x, T, cache, host)
        _, hits, missing, evicted = oracle.call(touched)
        print("  [cache] call %d batch %d: touched %d, hits %d, misses %d, evicted %d"
              % (n, b, len(touched), hits, len(missing), len(evicted)), flush=True)
        assert np.array_equal(o1, o2), n
        cache.check(mq, oracle)
    assert oracle.misses > 128 and oracle.hits > 0            # evictions happened, and hits
    if policy == 1:
        assert oracle.uncached > 0                            # misses the admission rule turned away


@pytest.mark.parametrize("q4", [(False, False), (True, True), (False, True)], ids=["q2", "q4", "q4dn"])
def test_cache_prefill_and_one_token(q4):
    """The prefill kernels (300 tokens: all experts touched, the cache holds the whole
    layer) and a one-token call on the same cache; 2-bit experts, 4-bit experts, and
    a 4-bit down matrix only (the prefill kernels' 64-slot units)."""
    mq = need_gpu()
    from bit_quantized_routed_amd import workload as dw
    wl = W.Workload("cache_e32_t300", 41, 300, 512, 32, 4, 512, 256, "bf16", 0.05, q4_gu=q4[0], q4_down=q4[1])
    dl = dw.DeviceLayer(wl)
    host = _host_copy(dl.experts)
    cache = _Cache(mq, 32, 32, wl.expert_bytes)
    oracle = LRUCache(32)
    x = dw.activations(wl)
    assert mq.describe(dl.shape(0), 300, wl.topk)["routed_kernel"] == 2
    for T, xx in ((300, x), (1, x[7:8].contiguous()), (300, x)):
        o1, o2, touched = _pair(mq, dl, xx, T, cache, host)
        oracle.call(touched)
        assert np.array_equal(o1, o2), T
        cache.check(mq, oracle)


def test_cache_smaller_than_a_call():
    """A budget of 8 slots for calls touching ~60 experts: the first misses in key
    order are cached, the rest read straight from host memory by the routed kernels;
    the outputs are still the resident layer's bits."""
    mq = need_gpu()
    from bit_quantized_routed_amd import workload as dw
    wl = W.Workload("cache_e64_t24", 42, 24, 512, 64, 6, 512, 256, "bf16", 0.05, zipf=True)
    dl = dw.DeviceLayer(wl)
    host = _host_copy(dl.experts)
    cache = _Cache(mq, 8, 64, wl.expert_bytes)
    oracle = LRUCache(8)
    xs = dw.activations(wl, tokens=48)
    for b in (0, 1, 0):
        x = xs[24 * b:24 * (b + 1)].contiguous()
        o1, o2, touched = _pair(mq, dl, x, 24, cache, host)
        oracle.call(touched)
        print("  [cache] small budget: touched %d, uncached %d" % (len(touched), oracle.last_uncached), flush=True)
        assert oracle.last_uncached > 0
        assert np.array_equal(o1, o2), b
        cache.check(mq, oracle)


def test_cache_shared_by_two_layers():
    mq = need_gpu()
    from bit_quantized_routed_amd import workload as dw
    wl = W.WORKLOADS["tiny_stack"]
    layers = [dw.DeviceLayer(wl, layer=l) for l in range(2)]
    hosts = [_host_copy(l.experts) for l in layers]
    E = wl.n_experts
    cache = _Cache(mq, 12, 2 * E, wl.expert_bytes)        # 12 slots for 2 x 8 experts
    oracle = LRUCache(12)
    h = dw.layer_residual(wl, 0)
    for step in range(3):
        for l, (dl, host) in enumerate(zip(layers, hosts)):
            x = h[4 * step:4 * step + 4].contiguous()
            o1, o2, touched = _pair(mq, dl, x, 4, cache, host, key_base=l * E, flags=mq.RESIDUAL_ADD)
            oracle.call(touched + l * E)
            assert np.array_equal(o1, o2), (step, l)
            cache.check(mq, oracle)


def test_cache_under_graph_capture():
    """A captured cached forward replays the plan and the fill each time: outputs equal
    the resident layer's, and the state advances like the oracle's (hits only)."""
    mq = need_gpu()
    from bit_quantized_routed_amd import workload as dw
    wl = W.WORKLOADS["tiny"]
    dl = dw.DeviceLayer(wl)
    host = _host_copy(dl.experts)
    T, E = wl.tokens, wl.n_experts
    cache = _Cache(mq, 8, E, wl.expert_bytes)
    oracle = LRUCache(8)
    shape = dl.shape(0)
    ws = dw.workspace(shape, T, wl.topk)
    x = dw.activations(wl)
    ref, o, touched = _pair(mq, dl, x, T, cache, host)
    oracle.call(touched)
    out = torch.zeros((T, wl.hidden), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        mq.forward_cached(x, dl.router_w, host, 0, cache.c, dl.shared_w, wl.topk, out, shape, T,
                          router_b=dl.router_b, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    oracle.call(touched)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mq.forward_cached(x, dl.router_w, host, 0, cache.c, dl.shared_w, wl.topk, out, shape, T,
                          router_b=dl.router_b, workspace=ws)
    for rep in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        oracle.call(touched)
        assert np.array_equal(out.cpu().numpy(), ref), rep
        cache.check(mq, oracle)


@pytest.mark.parametrize("policy", [0, 1], ids=["lru", "lru_admit"])
def test_cache_clock_renumbering(policy):
    """When the call clock reaches its limit (2^30, set here from the host), the next
    call renumbers the used slots' stamps in (stamp, slot) order before it plans: the
    slot contents, key map, counters and every later eviction stay those of the
    oracle's policy, whose clock never wraps."""
    mq = need_gpu()
    from bit_quantized_routed_amd import workload as dw
    wl = W.Workload("cache_e32_t6", 43, 6, 512, 32, 4, 512, 0, "bf16", 0.05, zipf=True)
    dl = dw.DeviceLayer(wl)
    host = _host_copy(dl.experts)
    cache = _Cache(mq, 10, 32, wl.expert_bytes, policy=policy)
    oracle = LRUCache(10, admit=policy == 1)
    xs = dw.activations(wl, tokens=6 * 8)
    H, n = mq.CACHE_HDR, cache.n_slots

    def check_order():
        st = cache.state.cpu().numpy()
        key, stamp = st[H:H + n], st[H + n:H + 2 * n]
        key_slot, key_count = st[H + 2 * n:H + 2 * n + cache.n_keys], st[H + 2 * n + cache.n_keys:]
        assert key.tolist() == oracle.key
        assert all(key_count[k] == oracle.count.get(k, 0) for k in range(cache.n_keys))
        assert st[1] == oracle.hits and st[2] == oracle.misses and st[6] == oracle.uncached
        order_dev = sorted(range(n), key=lambda s: (stamp[s], s))
        order_ora = sorted(range(n), key=lambda s: (oracle.stamp[s], s))
        assert order_dev == order_ora
        assert all((stamp[s] == 0) == (oracle.stamp[s] == 0) for s in range(n))
        want = np.full(cache.n_keys, -1)
        for s, k in enumerate(oracle.key):
            if k >= 0:
                want[k] = s
        assert np.array_equal(key_slot, want)
        return int(st[0])

    for b in range(4):
        x = xs[6 * b:6 * (b + 1)].contiguous()
        o1, o2, touched = _pair(mq, dl, x, 6, cache, host)
        oracle.call(touched)
        assert np.array_equal(o1, o2), b
        cache.check(mq, oracle)
    cache.state[0] = 1 << 30                             # the clock at its limit
    torch.cuda.synchronize()
    for b in (4, 0, 5, 6, 1, 7):
        x = xs[6 * b:6 * (b + 1)].contiguous()
        o1, o2, touched = _pair(mq, dl, x, 6, cache, host)
        oracle.call(touched)
        assert np.array_equal(o1, o2), b
        clock = check_order()
        assert clock <= n + 6                            # renumbered, then counting again

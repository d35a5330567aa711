"""The seeded synthetic workloads and the stream layout of their tensors.

Shapes follow a DeepSeek-class MoE layer (hidden 7168, 256 routed experts,
top-8, expert intermediate 2048, one bf16 shared expert of intermediate 2048),
plus one tiny layer for exhaustive checks.  Every tensor is a pure function of
(seed, stream id, index); see gen.py for the value definition.

Stream id (64-bit): bits 32..47 = layer + 1 (0 for the activations), low 32 bits
= tensor code:
    1            activations x (or the initial residual stream h_0)
    2            router weights [E, H]
    3            router-bias permutation keys [E]
    4            a standalone residual-stream input of this layer [T, H] (fp32), for
                 checking each layer of a stack on its own input
    8, 9, 10     shared expert gate [Is, H], up [Is, H], down [H, Is]
    16 + 3e + m  routed expert e, matrix m (0 gate [I, H], 1 up [I, H], 2 down [H, I])
"""
import json
import math
import os
from dataclasses import dataclass

import numpy as np

from . import gen
from .philox import philox4x32_10

TENSOR_X = 1
TENSOR_ROUTER_W = 2
TENSOR_ROUTER_PERM = 3
TENSOR_H_LAYER = 4
TENSOR_SHARED = 8
TENSOR_EXPERT = 16


def stream_id(layer, tensor):
    if tensor == TENSOR_X:
        return TENSOR_X
    return ((int(layer) + 1) << 32) | int(tensor)


def expert_stream(layer, e, m):
    return stream_id(layer, TENSOR_EXPERT + 3 * int(e) + int(m))


_ALPHA_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "zipf_alpha.json")


def zipf_alpha():
    """Router-bias strength for Zipf(1.1) expert popularity (calibrated offline)."""
    with open(_ALPHA_FILE) as f:
        return float(json.load(f)["alpha"])


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    tokens: int
    hidden: int
    n_experts: int
    topk: int
    inter: int
    shared_inter: int          # 0: no shared expert
    act: str                   # "f32" or "bf16"
    router_sigma: float
    expert_sigma: float = 0.02
    shared_sigma: float = 0.02
    zipf: bool = False
    layers: int = 1
    rmsnorm: bool = False
    rms_eps: float = float(np.float32(1e-6))     # the fp32 value the library receives
    # routed matrices in the 4-bit sibling format: gate/up and/or down, in the layers
    # from q4_from on (the rest in the 2-bit format)
    q4_gu: bool = False
    q4_down: bool = False
    q4_from: int = 0

    @property
    def blocks_per_expert(self):
        return 3 * self.hidden * self.inter // 256

    def q4_at(self, layer):
        """(gate/up in Q4, down in Q4) for a layer."""
        on = layer >= self.q4_from
        return self.q4_gu and on, self.q4_down and on

    def expert_bytes_at(self, layer):
        gu, dn = self.q4_at(layer)
        nb = self.hidden * self.inter // 256
        return 2 * nb * (148 if gu else 84) + nb * (148 if dn else 84)

    @property
    def expert_bytes(self):
        """Bytes of one routed expert of layer 0."""
        return self.expert_bytes_at(0)

    def x_stream(self):
        return stream_id(0, TENSOR_X)


H_DS, E_DS, K_DS, I_DS = 7168, 256, 8, 2048

WORKLOADS = {
    "tiny": Workload("tiny", 0, 4, 256, 8, 2, 512, 0, "f32", 0.05),
    "decode1": Workload("decode1", 1, 1, H_DS, E_DS, K_DS, I_DS, I_DS, "bf16", 0.02),
    "decode32_zipf": Workload("decode32_zipf", 2, 32, H_DS, E_DS, K_DS, I_DS, I_DS, "bf16",
                              0.02, zipf=True),
    "prefill2048": Workload("prefill2048", 3, 2048, H_DS, E_DS, K_DS, I_DS, I_DS, "bf16",
                            1.0 / math.sqrt(H_DS)),
    "stack40_t64_zipf": Workload("stack40_t64_zipf", 4, 64, H_DS, E_DS, K_DS, I_DS, I_DS,
                                 "bf16", 0.02, zipf=True, layers=40, rmsnorm=True),
    # small residual stack for exhaustive checks of RMSNorm + residual over many layers
    "tiny_stack": Workload("tiny_stack", 5, 16, 256, 8, 2, 512, 256, "bf16", 0.05,
                           layers=12, rmsnorm=True),
    # speculative verification micro-batch: 16 sessions, each checking 5 draft tokens
    # plus its current one in one batched target pass (T = 16 x 6), Zipf routing
    "verify96_zipf": Workload("verify96_zipf", 6, 96, H_DS, E_DS, K_DS, I_DS, I_DS, "bf16",
                              0.02, zipf=True),
    # the deep stack with its last 6 expert layers in the 4-bit sibling format (layers
    # 0..33 are those of stack40_t64_zipf: same seed)
    "stack40_q2q4": Workload("stack40_q2q4", 4, 64, H_DS, E_DS, K_DS, I_DS, I_DS, "bf16", 0.02,
                             zipf=True, layers=40, rmsnorm=True, q4_gu=True, q4_down=True, q4_from=34),
    # the prefill layer with both routed matrices in the 4-bit sibling format (the
    # same seed: prefill2048's activations, router and routing)
    "prefill2048_q4": Workload("prefill2048_q4", 3, 2048, H_DS, E_DS, K_DS, I_DS, I_DS, "bf16",
                               1.0 / math.sqrt(H_DS), q4_gu=True, q4_down=True),
    # the one-token decode layer with both routed matrices in the 4-bit format
    "decode1_q4": Workload("decode1_q4", 1, 1, H_DS, E_DS, K_DS, I_DS, I_DS, "bf16", 0.02,
                           q4_gu=True, q4_down=True),
    # tiny layers in the 4-bit format: both matrices, and gate/up only (per-matrix mix)
    "tiny_q4": Workload("tiny_q4", 7, 4, 256, 8, 2, 512, 256, "bf16", 0.05, q4_gu=True, q4_down=True),
    "tiny_q4gu": Workload("tiny_q4gu", 8, 5, 256, 8, 2, 512, 0, "f32", 0.05, q4_gu=True),
    # mid-size layers (hidden and intermediate 2048, 64 experts, top-8, 24 tokens, Zipf) for
    # option combinations: a one-token call splits the reduction, a 24-token call need not
    "mid_e64": Workload("mid_e64", 51, 24, 2048, 64, 8, 2048, 256, "bf16", 0.05, zipf=True),
    "mid_e64_q4": Workload("mid_e64_q4", 52, 24, 2048, 64, 8, 2048, 256, "bf16", 0.05, zipf=True,
                           q4_gu=True, q4_down=True),
    "mid_e64_q4gu": Workload("mid_e64_q4gu", 53, 24, 2048, 64, 8, 2048, 0, "bf16", 0.05, zipf=True,
                             q4_gu=True),
    "mid_e64_q4dn": Workload("mid_e64_q4dn", 54, 24, 2048, 64, 8, 2048, 256, "bf16", 0.05, zipf=True,
                             q4_down=True),
}
ORDER = ["tiny", "decode1", "decode32_zipf", "prefill2048", "stack40_t64_zipf"]


# ---------------------------------------------------------------- host tensors
def _normal(wl, stream, n, sigma, start=0):
    from . import normal_f32          # C generator (same values as gen.normal_f32)
    return normal_f32(wl.seed, stream, n, sigma, start)


def activations(wl, tokens=None, start_token=0):
    """x [T, H]: fp32 N(0,1) values; for bf16 workloads rounded to bf16 (values
    returned as fp32 holding bf16 values, plus the uint16 bits)."""
    T = wl.tokens if tokens is None else tokens
    v = _normal(wl, wl.x_stream(), T * wl.hidden, 1.0, start_token * wl.hidden)
    v = v.reshape(T, wl.hidden)
    if wl.act == "bf16":
        bits = gen.f32_to_bf16_bits(v)
        return gen.bf16_bits_to_f32(bits), bits
    return v, None


def layer_residual(wl, layer, tokens=None):
    """A residual-stream input of one layer of a stack [T, H]: fp32 N(0,1) draws of
    the layer's own stream (not bf16-rounded: RMSNorm sees a full fp32 stream)."""
    T = wl.tokens if tokens is None else tokens
    return _normal(wl, stream_id(layer, TENSOR_H_LAYER), T * wl.hidden, 1.0).reshape(T, wl.hidden)


def router_weights(wl, layer=0):
    return _normal(wl, stream_id(layer, TENSOR_ROUTER_W), wl.n_experts * wl.hidden,
                   wl.router_sigma).reshape(wl.n_experts, wl.hidden)


def router_rank(wl, layer=0):
    """r_e in 1..E: popularity rank of expert e (a seeded permutation)."""
    s = stream_id(layer, TENSOR_ROUTER_PERM)
    idx = np.arange(wl.n_experts, dtype=np.uint64)
    k0, k1 = wl.seed & 0xFFFFFFFF, (wl.seed >> 32) & 0xFFFFFFFF
    keys = philox4x32_10(idx, 0, s & 0xFFFFFFFF, s >> 32, k0, k1)[0]
    order = np.argsort(keys, kind="stable")
    rank = np.empty(wl.n_experts, dtype=np.int64)
    rank[order] = np.arange(1, wl.n_experts + 1)
    return rank


def router_bias(wl, layer=0, alpha=None):
    """b_e = -alpha * ln(r_e) (fp32) for Zipf workloads, else None."""
    if not wl.zipf:
        return None
    a = zipf_alpha() if alpha is None else alpha
    return (-a * np.log(router_rank(wl, layer).astype(np.float64))).astype(np.float32)


def shared_bf16_bits(wl, layer=0):
    """Shared expert (gate [Is,H], up [Is,H], down [H,Is]) as bf16 bit patterns."""
    if not wl.shared_inter:
        return None
    Is, H = wl.shared_inter, wl.hidden
    shapes = [(Is, H), (Is, H), (H, Is)]
    out = []
    for m, shp in enumerate(shapes):
        v = _normal(wl, stream_id(layer, TENSOR_SHARED + m), shp[0] * shp[1], wl.shared_sigma)
        out.append(gen.f32_to_bf16_bits(v).reshape(shp))
    return tuple(out)


def expert_f32(wl, layer, e, m):
    """Routed expert e, matrix m (0 gate, 1 up, 2 down) as fp32 N(0, 0.02^2) draws."""
    rows, cols = (wl.inter, wl.hidden) if m < 2 else (wl.hidden, wl.inter)
    v = _normal(wl, expert_stream(layer, e, m), rows * cols, wl.expert_sigma)
    return v.reshape(rows, cols)

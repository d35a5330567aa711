"""Device-side materialisation of the seeded synthetic workloads (tests, bench).

Every tensor is drawn on the GPU with moe_q2_synth_normal from the same
(seed, stream, index) definition as the host generator in `synth`, and routed
expert matrices are encoded with moe_q2_quantize.  The router bias (E floats,
a logarithm of seeded ranks) is made on the host and uploaded.
"""
import numpy as np
import torch

from synth import workloads as W
from synth.gen import normal_scale

from . import (BF16, F32, GU_Q4, DOWN_Q4, PRE_RMSNORM, make_shape, quantize, quantize_q4, synth_normal,
               workspace_size, pack_expert)


def _normal(wl, stream_id, n, sigma, dtype, out=None, start=0):
    dev = torch.device("cuda")
    if out is None:
        out = torch.empty(n, dtype=torch.float32 if dtype == F32 else torch.bfloat16, device=dev)
    synth_normal(wl.seed, stream_id, start, n, float(normal_scale(sigma)), out, out_dtype=dtype)
    return out


class DeviceLayer:
    """Weights of one layer of a workload, resident in HBM."""

    def __init__(self, wl, layer=0, tmp=None, experts_out=None):
        self.wl, self.layer = wl, layer
        E, H, I = wl.n_experts, wl.hidden, wl.inter
        self.router_w = _normal(wl, W.stream_id(layer, W.TENSOR_ROUTER_W), E * H,
                                wl.router_sigma, F32).view(E, H)
        b = W.router_bias(wl, layer)
        self.router_b = None if b is None else torch.from_numpy(b).cuda()
        self.shared_w = None
        if wl.shared_inter:
            Is = wl.shared_inter
            self.shared_w = torch.empty(3 * Is * H, dtype=torch.bfloat16, device="cuda")
            for m in range(3):
                _normal(wl, W.stream_id(layer, W.TENSOR_SHARED + m), Is * H, wl.shared_sigma, BF16,
                        out=self.shared_w[m * Is * H:(m + 1) * Is * H])
        gu4, dn4 = wl.q4_at(layer)
        self.codec_flags = (GU_Q4 if gu4 else 0) | (DOWN_Q4 if dn4 else 0)
        ebytes = wl.expert_bytes_at(layer)
        self.expert_bytes = ebytes
        self.experts = experts_out if experts_out is not None else \
            torch.empty(E * ebytes, dtype=torch.uint8, device="cuda")
        if tmp is None:
            tmp = torch.empty(H * I, dtype=torch.float32, device="cuda")
        nb = H * I // 256
        mb = [nb * (148 if gu4 else 84)] * 2 + [nb * (148 if dn4 else 84)]      # bytes per matrix
        off = [0, mb[0], mb[0] + mb[1], ebytes]
        rm = torch.empty(ebytes, dtype=torch.uint8, device="cuda")     # row-major staging
        shp = self.shape()
        for e in range(E):
            for m in range(3):
                _normal(wl, W.expert_stream(layer, e, m), H * I, wl.expert_sigma, F32, out=tmp)
                rows, k = (I, H) if m < 2 else (H, I)
                q4 = gu4 if m < 2 else dn4
                (quantize_q4 if q4 else quantize)(tmp, rows, k, rm[off[m]:off[m + 1]])
            pack_expert(rm[off[0]:off[1]], rm[off[1]:off[2]], rm[off[2]:off[3]], shp,
                        self.experts[e * ebytes:(e + 1) * ebytes])
        del rm

    def shape(self, flags=0):
        """The layer's shape descriptor: its activation type, RMSNorm for a residual
        stack, its weight formats, plus `flags`."""
        wl = self.wl
        act = BF16 if wl.act == "bf16" else F32
        if wl.rmsnorm:
            flags |= PRE_RMSNORM
        gu4, dn4 = wl.q4_at(self.layer)
        flags |= (GU_Q4 if gu4 else 0) | (DOWN_Q4 if dn4 else 0)
        return make_shape(wl.hidden, wl.inter, wl.n_experts, wl.shared_inter, act, flags,
                          wl.rms_eps)


def activations(wl, tokens=None):
    """x [T, H] on the device: fp32, or bf16 for bf16 workloads;
    for the residual stack this is the initial residual stream (fp32 holding bf16 values)."""
    T = wl.tokens if tokens is None else tokens
    n = T * wl.hidden
    sid = W.stream_id(0, W.TENSOR_X)
    if wl.rmsnorm:
        return _normal(wl, sid, n, 1.0, BF16).float().view(T, wl.hidden).contiguous()
    if wl.act == "bf16":
        return _normal(wl, sid, n, 1.0, BF16).view(T, wl.hidden)
    return _normal(wl, sid, n, 1.0, F32).view(T, wl.hidden)


def layer_residual(wl, layer, tokens=None):
    """The standalone residual-stream input of one stack layer [T, H] fp32 (the
    device twin of synth.workloads.layer_residual)."""
    T = wl.tokens if tokens is None else tokens
    return _normal(wl, W.stream_id(layer, W.TENSOR_H_LAYER), T * wl.hidden, 1.0, F32).view(T, wl.hidden)


def workspace(shape, tokens, topk):
    n = workspace_size(shape, tokens, topk)
    return torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")

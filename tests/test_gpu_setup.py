"""GPU: the device generator and the device quantizer reproduce the host
generator and the oracle's quantizer bit for bit."""
import numpy as np
import pytest
import torch

import synth
from oracle import q2, q4
from synth import workloads as W
from synth.gen import normal_scale, f32_to_bf16_bits
from tests.gpu_util import need_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("seed,stream,start,n,sigma", [
    (0, 1, 0, 1000, 1.0), (3, (7 << 32) | 16, 12345, 100003, 0.02), (2**33 + 5, 2, 2**34, 4096, 0.5)])
def test_device_normal_matches_host(seed, stream, start, n, sigma):
    mq = need_gpu()
    out = torch.empty(n, dtype=torch.float32, device="cuda")
    mq.synth_normal(seed, stream, start, n, float(normal_scale(sigma)), out)
    host = synth.normal_f32(seed, stream, n, sigma, start)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), host.view(np.uint32))
    ob = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    mq.synth_normal(seed, stream, start, n, float(normal_scale(sigma)), ob, out_dtype=mq.BF16)
    assert np.array_equal(ob.view(torch.int16).cpu().numpy().view(np.uint16), f32_to_bf16_bits(host))


def _dev_quant(mq, w_np, q4_codec=False):
    w = torch.from_numpy(np.ascontiguousarray(w_np, dtype=np.float32)).cuda()
    nb = w.numel() // 256
    bb = 148 if q4_codec else 84
    out = torch.empty(nb * bb, dtype=torch.uint8, device="cuda")
    (mq.quantize_q4 if q4_codec else mq.quantize)(w, nb, 256, out)
    return out.cpu().numpy().reshape(nb, bb)


def test_device_quantizer_matches_oracle_edges():
    mq = need_gpu()
    rng = np.random.default_rng(0)
    blocks = [np.zeros(256), np.full(256, -0.375), np.full(256, 3.0),
              np.abs(rng.standard_normal(256)) + 0.01, -np.abs(rng.standard_normal(256)),
              rng.standard_normal(256) * 1e-3, rng.standard_normal(256) * 50,
              np.where(np.arange(256) % 16 == 0, 1.0, 0.0), rng.standard_normal(256) * 2.0 ** -20]
    w = np.stack(blocks).astype(np.float32)
    assert np.array_equal(_dev_quant(mq, w), q2.encode_blocks(w))
    assert np.array_equal(_dev_quant(mq, w, True), q4.encode_blocks(w))


@pytest.mark.parametrize("name,e,m", [("tiny", 0, 0), ("tiny", 7, 2), ("decode1", 5, 1),
                                      ("decode32_zipf", 200, 2)])
def test_device_quantizer_matches_oracle_on_workload(name, e, m):
    mq = need_gpu()
    wl = W.WORKLOADS[name]
    w = W.expert_f32(wl, 0, e, m)
    assert np.array_equal(_dev_quant(mq, w), q2.encode_matrix(w))
    assert np.array_equal(_dev_quant(mq, w, True), q4.encode_matrix(w))


@pytest.mark.parametrize("name,layer", [("decode1", 0), ("stack40_q2q4", 39), ("tiny_q4gu", 0)])
def test_device_pack_matches_oracle_layout(name, layer):
    """The device packer against the oracle's layout, for the 2-bit expert, the 4-bit
    one and the per-matrix mix (gate/up in 4 bits, down in 2)."""
    mq = need_gpu()
    from bit_quantized_routed_amd import workload as dw
    from tests.oracle_inputs import HostLayer
    wl = W.WORKLOADS[name]
    hl = HostLayer(wl, layer)
    g, u, d = hl.expert_bytes(3)
    dev = [torch.from_numpy(np.ascontiguousarray(a).reshape(-1)).cuda() for a in (g, u, d)]
    out = torch.empty(wl.expert_bytes_at(layer), dtype=torch.uint8, device="cuda")
    gu4, dn4 = wl.q4_at(layer)
    shape = mq.make_shape(wl.hidden, wl.inter, wl.n_experts, 0,
                          flags=(mq.GU_Q4 if gu4 else 0) | (mq.DOWN_Q4 if dn4 else 0))
    mq.pack_expert(dev[0], dev[1], dev[2], shape, out)
    assert np.array_equal(out.cpu().numpy(), hl.packed_expert(3))

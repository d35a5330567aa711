"""GPU: the device generator and the device quantizer reproduce the host
generator and the oracle's quantizer bit for bit."""
import numpy as np
import pytest
import torch

import synth
from oracle import q2
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


def _dev_quant(mq, w_np):
    w = torch.from_numpy(np.ascontiguousarray(w_np, dtype=np.float32)).cuda()
    nb = w.numel() // 256
    out = torch.empty(nb * 84, dtype=torch.uint8, device="cuda")
    mq.quantize(w, nb, 256, out)
    return out.cpu().numpy().reshape(nb, 84)


def test_device_quantizer_matches_oracle_edges():
    mq = need_gpu()
    rng = np.random.default_rng(0)
    blocks = [np.zeros(256), np.full(256, -0.375), np.full(256, 3.0),
              np.abs(rng.standard_normal(256)) + 0.01, -np.abs(rng.standard_normal(256)),
              rng.standard_normal(256) * 1e-3, rng.standard_normal(256) * 50,
              np.where(np.arange(256) % 16 == 0, 1.0, 0.0), rng.standard_normal(256) * 2.0 ** -20]
    w = np.stack(blocks).astype(np.float32)
    assert np.array_equal(_dev_quant(mq, w), q2.encode_blocks(w))


@pytest.mark.parametrize("name,e,m", [("tiny", 0, 0), ("tiny", 7, 2), ("decode1", 5, 1),
                                      ("decode32_zipf", 200, 2)])
def test_device_quantizer_matches_oracle_on_workload(name, e, m):
    mq = need_gpu()
    wl = W.WORKLOADS[name]
    w = W.expert_f32(wl, 0, e, m)
    assert np.array_equal(_dev_quant(mq, w), q2.encode_matrix(w))


def test_device_pack_matches_oracle_layout():
    mq = need_gpu()
    from bit_quantized_routed_amd import workload as dw
    from tests.oracle_inputs import host_layer
    wl = W.WORKLOADS["decode1"]
    hl = host_layer("decode1")
    g, u, d = hl.expert_bytes(3)
    dev = [torch.from_numpy(np.ascontiguousarray(a).reshape(-1)).cuda() for a in (g, u, d)]
    out = torch.empty(wl.expert_bytes, dtype=torch.uint8, device="cuda")
    mq.pack_expert(dev[0], dev[1], dev[2], wl.hidden, wl.inter, out)
    assert np.array_equal(out.cpu().numpy(), hl.packed_expert(3))

"""Seeded input generator: Philox4x32-10 against its published known-answer
vectors (Random123 distribution, kat_vectors), C vs NumPy bit identity, moments."""
import numpy as np
import pytest

import synth
from synth import gen, workloads
from synth.philox import philox4x32_10

# (counter, key, expected output) -- Salmon et al. SC'11 reference implementation KAT.
KAT = [
    ((0, 0, 0, 0), (0, 0), (0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8)),
    ((0xffffffff,) * 4, (0xffffffff, 0xffffffff), (0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd)),
    ((0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344), (0xa4093822, 0x299f31d0),
     (0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1)),
]


@pytest.mark.parametrize("ctr,key,want", KAT)
def test_philox_kat_numpy(ctr, key, want):
    got = tuple(int(v) for v in philox4x32_10(*ctr, *key))
    assert got == want


@pytest.mark.parametrize("ctr,key,want", KAT)
def test_philox_kat_c(ctr, key, want):
    assert tuple(int(v) for v in synth.philox_c(ctr, key)) == want


def test_c_matches_numpy_bits():
    for seed, stream, start in [(0, 1, 0), (3, (5 << 32) | 77, 123456789), (2**40 + 7, 2, 2**33)]:
        a = gen.normal_f32(seed, stream, 50000, 0.02, start)
        b = synth.normal_f32(seed, stream, 50000, 0.02, start)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_moments_and_support():
    v = synth.normal_f32(9, 4, 1 << 20, 0.5).astype(np.float64)
    assert abs(v.mean()) < 0.5 * 5e-3
    assert abs(v.std() / 0.5 - 1) < 5e-3
    # Irwin-Hall(8) is bounded: |S - mean| <= 262140, i.e. 4.899 sd
    assert np.abs(v).max() <= 0.5 * 262140 / gen.IH_SD * (1 + 1e-6)


def test_bf16_rounding_ties_to_even():
    vals = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-8 + 2**-20, -1.0 - 2**-8],
                    dtype=np.float32)
    want = np.array([1.0, 1.0, 1.0 + 2**-6, 1.0 + 2**-7, -1.0], dtype=np.float32)
    got = gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(vals))
    assert np.array_equal(got, want)


def test_stream_ids_distinct():
    wl = workloads.WORKLOADS["decode1"]
    ids = {workloads.stream_id(0, workloads.TENSOR_X)}
    for layer in range(40):
        for t in (workloads.TENSOR_ROUTER_W, workloads.TENSOR_ROUTER_PERM, 8, 9, 10):
            ids.add(workloads.stream_id(layer, t))
        for e in range(wl.n_experts):
            for m in range(3):
                ids.add(workloads.expert_stream(layer, e, m))
    assert len(ids) == 1 + 40 * (5 + wl.n_experts * 3)


def test_zipf_rank_is_permutation():
    wl = workloads.WORKLOADS["decode32_zipf"]
    r = workloads.router_rank(wl)
    assert sorted(r.tolist()) == list(range(1, wl.n_experts + 1))
    b = workloads.router_bias(wl)
    assert b.dtype == np.float32 and b[np.argmin(r)] == 0.0

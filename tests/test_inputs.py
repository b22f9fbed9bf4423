"""Pins for the seeded input generator (fa_inputs): published test vector,
counter addressing, rounding against independent library conversions, and
the distribution's moments."""

import math

import numpy as np
import pytest
import torch

import fa_inputs as fi


def test_splitmix64_published_vector():
    # First five outputs of SplitMix64 seeded with 1234567, as published with
    # the generator's reference implementation (e.g. the Rosetta Code task
    # "Pseudo-random numbers/Splitmix64").
    want = [6457827717110365317, 3203168211198807973, 9817491932198370423,
            4593380528125082431, 16408922859458223821]
    got = [int(x) for x in fi.splitmix64_at(1234567, np.arange(5))]
    assert got == want


def test_splitmix64_matches_sequential_python():
    # an independent sequential pure-Python implementation of the same generator
    def seq(seed, n):
        x = seed
        out = []
        for _ in range(n):
            x = (x + fi.GAMMA) & ((1 << 64) - 1)
            z = x
            z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & ((1 << 64) - 1)
            z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & ((1 << 64) - 1)
            out.append(z ^ (z >> 31))
        return out

    for seed in (0, 1, 2**63 + 12345, 2**64 - 1):
        assert [int(x) for x in fi.splitmix64_at(seed, np.arange(50))] == seq(seed, 50)


def test_counter_addressing_independent_of_chunking():
    a = fi.tensor_bits(7, "k", (3, 1000), "f16", chunk=1 << 22)
    b = fi.tensor_bits(7, "k", (3, 1000), "f16", chunk=37)
    assert np.array_equal(a, b)
    key = fi.stream_key(7, fi.TENSOR_IDS["k"])
    x = fi.normals(key, 1234, 10)
    y = fi.normals(key, 0, 1244)[1234:]
    assert np.array_equal(x, y)


def test_streams_differ_and_are_deterministic():
    q1 = fi.tensor_bits(3, "q", (4096,), "bf16")
    q2 = fi.tensor_bits(3, "q", (4096,), "bf16")
    k1 = fi.tensor_bits(3, "k", (4096,), "bf16")
    q4 = fi.tensor_bits(4, "q", (4096,), "bf16")
    assert np.array_equal(q1, q2)
    assert not np.array_equal(q1, k1)
    assert not np.array_equal(q1, q4)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_rounding_matches_torch(dtype):
    rng = np.random.default_rng(0)
    # random bit patterns over the finite float32 range, plus exact ties
    bits = rng.integers(0, 2**32, size=200_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    ties = (np.arange(1, 5000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties, np.array([0.0, -0.0, 65504.0, 65520.0, 1e-8], np.float32)])
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    want = torch.from_numpy(x).to(tdt).view(torch.int16).numpy().view(np.uint16)
    got = fi.f32_to_bits(x, dtype)
    assert np.array_equal(got, want)


def test_normal_moments():
    n = 1 << 20
    x = fi.normals(fi.stream_key(11, 0), 0, n)
    se = 1.0 / math.sqrt(n)
    assert abs(x.mean()) < 5 * se
    assert abs(x.var() - 1.0) < 5 * math.sqrt(2.0) * se
    # fraction inside one standard deviation: 0.682689...
    frac = np.mean(np.abs(x) < 1.0)
    assert abs(frac - 0.6826894921) < 5 * math.sqrt(0.6827 * 0.3173 / n)
    assert np.all(np.isfinite(x))


def test_workload_counts():
    w = fi.WORKLOADS["causal_b2h8_s1024_d64_f16"]
    assert w.unmasked_pairs() == 1024 * 1025 // 2
    assert w.flops() == 4 * 2 * 8 * 64 * (1024 * 1025 // 2)
    w = fi.WORKLOADS["b2h32_s8192_d64_f16"]
    assert w.flops() == 4 * 2 * 32 * 64 * 8192 * 8192
    # Sq > Sk causal: rows past Sk see every key
    w2 = fi.Workload("x", 1, 1, 10, 4, 64, "f16", True, 0)
    assert w2.unmasked_pairs() == sum(min(i + 1, 4) for i in range(10))

"""Pins for the float64 GEMM + bias + GELU oracle: textbook values of the
normal distribution function, the identity gelu(x) - gelu(-x) = x, special
cases, the pre-activation against numpy's matmul, and the whole expression
against torch's float64 gelu(a @ w.T + b).  A dropped bias, a transposed
weight, a wrong GELU form (tanh instead of erf, missing 1/sqrt(2)) each fail
one of them."""

import math

import numpy as np
import pytest
import torch

import fa_inputs as fi


@pytest.fixture(scope="module")
def go():
    import oracle
    import oracle.gemm as g

    g._load()
    return g


def _dec(bits, dtype):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.float16 if dtype == "f16" else torch.bfloat16).double().numpy()


# Phi(x) from normal distribution tables (20 significant digits)
PHI = {0.5: 0.69146246127401310364, 1.0: 0.84134474606854293129, 2.0: 0.97724986805182079282,
       3.0: 0.99865010196837000638, -1.0: 0.15865525393145706871, -2.0: 0.02275013194817920718}


@pytest.mark.parametrize("x", sorted(PHI))
def test_gelu_table_values(go, x):
    assert go.gelu(x) == pytest.approx(x * PHI[x], rel=1e-14)


def test_gelu_identities(go):
    assert go.gelu(0.0) == 0.0
    for x in np.linspace(-8.0, 8.0, 161):
        assert go.gelu(x) - go.gelu(-x) == pytest.approx(x, rel=1e-13, abs=1e-15)
    assert go.gelu(12.0) == 12.0                         # Phi(12) rounds to 1
    assert -1e-30 < go.gelu(-12.0) <= 0.0                # -12 * Phi(-12) ~ -2e-32 (1 + erf cancels to 0)
    assert go.gelu(-5.0) == pytest.approx(-5.0 * 2.8665157187919391e-07, rel=1e-8)  # table Phi(-5)
    # not the tanh approximation: the two differ by ~1e-4 near |x| = 2
    x = 2.0
    tanh_form = 0.5 * x * (1 + math.tanh(math.sqrt(2 / math.pi) * (x + 0.044715 * x ** 3)))
    assert abs(go.gelu(x) - tanh_form) > 1e-5


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_pre_activation_is_matmul_plus_bias(go, dtype):
    M, N, K = 37, 29, 70
    a = fi.tensor_bits(51, "a", (M, K), dtype)
    w = fi.tensor_bits(51, "w", (N, K), dtype)
    b = fi.tensor_bits(51, "bias", (N,), dtype)
    c, pre = go.gemm_rows(a, w, b, dtype, want_pre=True)
    want = _dec(a, dtype) @ _dec(w, dtype).T + _dec(b, dtype)
    np.testing.assert_allclose(pre, want, rtol=1e-12, atol=1e-12)
    assert c.shape == (M, N)


def test_against_torch_float64(go):
    dtype = "bf16"
    M, N, K = 64, 48, 96
    a = fi.tensor_bits(52, "a", (M, K), dtype)
    w = fi.tensor_bits(52, "w", (N, K), dtype)
    b = fi.tensor_bits(52, "bias", (N,), dtype)
    c = go.gemm_rows(a, w, b, dtype, threads=4)
    ta, tw, tb = (torch.from_numpy(_dec(x, dtype)) for x in (a, w, b))
    ref = torch.nn.functional.gelu(ta @ tw.T + tb).numpy()
    np.testing.assert_allclose(c, ref, rtol=1e-12, atol=1e-13)


def test_identity_weight_and_zero_input(go):
    dtype = "f16"
    K = 16
    a = fi.tensor_bits(53, "a", (5, K), dtype)
    w = fi.f32_to_bits(np.eye(K, dtype=np.float32), dtype)
    b = fi.tensor_bits(53, "bias", (K,), dtype)
    c, pre = go.gemm_rows(a, w, b, dtype, want_pre=True)
    np.testing.assert_array_equal(pre, _dec(a, dtype) + _dec(b, dtype))
    z = np.zeros((3, K), np.uint16)
    cz = go.gemm_rows(z, w, b, dtype)
    want = np.array([go.gelu(x) for x in _dec(b, dtype)])
    np.testing.assert_array_equal(cz, np.broadcast_to(want, (3, K)))


def test_no_bias_and_row_subsets(go):
    dtype = "bf16"
    M, N, K = 40, 24, 40
    a = fi.tensor_bits(54, "a", (M, K), dtype)
    w = fi.tensor_bits(54, "w", (N, K), dtype)
    c0 = go.gemm_rows(a, w, None, dtype)
    cz = go.gemm_rows(a, w, np.zeros(N, np.uint16), dtype)
    np.testing.assert_array_equal(c0, cz)
    rows = np.array([39, 0, 17, 17], np.int64)
    np.testing.assert_array_equal(go.gemm_rows(a, w, None, dtype, rows=rows, threads=2), c0[rows])

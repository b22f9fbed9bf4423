"""Pins for the float64 row-wise oracles: the row softmax and the fused
RMSNorm + SiLU.  Closed forms, invariants and torch's float64 routines; a
missing max shift, a wrong normaliser, a mean replaced by a sum or a
sigmoid in place of SiLU each fail one of them."""

import math

import numpy as np
import pytest
import torch

import fa_inputs as fi


@pytest.fixture(scope="module")
def ro():
    import oracle.rowwise as r

    r._load()
    return r


def _dec(bits, dtype):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.float16 if dtype == "f16" else torch.bfloat16).double().numpy()


# --- softmax -----------------------------------------------------------------


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_softmax_rows_sum_to_one_and_match_torch(ro, dtype):
    x = fi.tensor_bits(71, "x", (37, 301), dtype, 3.0)
    y = ro.softmax_rows(x, dtype, threads=4)
    np.testing.assert_allclose(y.sum(1), 1.0, rtol=1e-14)
    assert np.all(y > 0) and np.all(y <= 1)
    ref = torch.softmax(torch.from_numpy(_dec(x, dtype)), dim=1).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-300)


def test_softmax_closed_forms(ro):
    dtype = "f16"
    # two entries: the logistic function of the difference
    x = fi.f32_to_bits(np.array([[1.0, -1.0], [0.0, 0.0], [5.0, 2.0]], np.float32), dtype)
    y = ro.softmax_rows(x, dtype)
    sig2 = 0.88079707797788244406  # 1 / (1 + e^-2), table value
    np.testing.assert_allclose(y[0], [sig2, 1 - sig2], rtol=1e-15)
    np.testing.assert_allclose(y[1], [0.5, 0.5], rtol=1e-15)
    sig3 = 0.95257412682243321912  # 1 / (1 + e^-3)
    np.testing.assert_allclose(y[2], [sig3, 1 - sig3], rtol=1e-15)
    # a constant row is uniform; huge values do not overflow
    c = fi.f32_to_bits(np.full((2, 1000), 60000.0, np.float32), dtype)
    np.testing.assert_allclose(ro.softmax_rows(c, dtype), 1e-3, rtol=1e-14)


def test_softmax_shift_invariance(ro):
    dtype = "bf16"
    rng = np.random.default_rng(1)
    v = rng.integers(-20, 20, size=(5, 64)).astype(np.float32)
    y1 = ro.softmax_rows(fi.f32_to_bits(v, dtype), dtype)
    y2 = ro.softmax_rows(fi.f32_to_bits(v + 37.0, dtype), dtype)
    np.testing.assert_allclose(y1, y2, rtol=1e-13)


# --- RMSNorm + SiLU ------------------------------------------------------------


def test_silu_values(ro):
    assert ro.silu(0.0) == 0.0
    assert ro.silu(1.0) == pytest.approx(0.73105857863000487925, rel=1e-15)   # logistic(1), table value
    assert ro.silu(-2.0) == pytest.approx(-2 * 0.11920292202211755594, rel=1e-14)  # -2 logistic(-2)
    for z in np.linspace(-10, 10, 101):
        assert ro.silu(z) - ro.silu(-z) == pytest.approx(z, rel=1e-13, abs=1e-15)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_rmsnorm_silu_matches_torch(ro, dtype):
    R, C, eps = 23, 640, 1e-6
    x = fi.tensor_bits(72, "x", (R, C), dtype, 2.0)
    g = fi.tensor_bits(72, "g", (C,), dtype)
    y, z = ro.rmsnorm_silu_rows(x, g, dtype, eps, threads=3, want_z=True)
    tx, tg = torch.from_numpy(_dec(x, dtype)), torch.from_numpy(_dec(g, dtype))
    zr = torch.nn.functional.rms_norm(tx, (C,), tg, eps)
    np.testing.assert_allclose(z, zr.numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(y, torch.nn.functional.silu(zr).numpy(), rtol=1e-12, atol=1e-14)


def test_rmsnorm_invariants(ro):
    dtype = "bf16"
    R, C = 6, 256
    x = fi.tensor_bits(73, "x", (R, C), dtype)
    ones = fi.f32_to_bits(np.ones(C, np.float32), dtype)
    # unit weight, eps 0: each normalised row has mean square 1
    _, z = ro.rmsnorm_silu_rows(x, ones, dtype, 0.0, want_z=True)
    np.testing.assert_allclose((z ** 2).mean(1), 1.0, rtol=1e-13)
    # scaling a row by 2 (exact) leaves it unchanged at eps 0
    x2 = fi.f32_to_bits(2 * _dec(x, dtype).astype(np.float32), dtype)
    _, z2 = ro.rmsnorm_silu_rows(x2, ones, dtype, 0.0, want_z=True)
    np.testing.assert_allclose(z2, z, rtol=1e-14)
    # eps enters under the root: mean square ms / (ms + eps)
    eps = 0.5
    _, ze = ro.rmsnorm_silu_rows(x, ones, dtype, eps, want_z=True)
    ms = (_dec(x, dtype) ** 2).mean(1)
    np.testing.assert_allclose((ze ** 2).mean(1), ms / (ms + eps), rtol=1e-13)

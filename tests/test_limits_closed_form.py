"""The closed form used by the largest-key-count GPU test, checked against a
plain float64 softmax over explicit scores on small key counts."""

import math

import numpy as np
import pytest

from test_gpu_limits import _expected, _sum_s


@pytest.mark.parametrize("Sk", [5, 8, 33, 1000, 1003])
def test_sum_of_quarter_index(Sk):
    j = np.arange(Sk)
    s = (4 * j) // Sk
    for a, b in [(0, Sk), (0, 3 * Sk // 4 + 1), (Sk // 3, Sk), (2, 3)]:
        assert _sum_s(a, b, Sk) == int(s[a:b].sum())


@pytest.mark.parametrize("Sk,D", [(1000, 8), (1003, 16), (64, 4)])
def test_two_level_softmax_closed_form(Sk, D):
    j1 = 3 * Sk // 4 + 7
    j = np.arange(Sk)
    v = ((4 * j) // Sk)[:, None] * ((np.arange(D) % 4) - 1.5)[None, :]
    k = np.zeros((Sk, D))
    k[j1:, 0] = 1.0
    q = np.zeros(D)
    q[0] = 48.0
    s = 0.125 * (k @ q)
    p = np.exp(s - s.max())
    o = (p @ v) / p.sum()
    lse = s.max() + math.log(p.sum())
    o_cf, lse_cf = _expected(Sk, D, j1)
    assert np.allclose(o_cf, o, rtol=1e-12, atol=1e-12)
    assert abs(lse_cf - lse) <= 1e-12 * abs(lse)

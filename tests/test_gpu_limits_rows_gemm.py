"""GEMM + bias + GELU and the row-wise kernels at their largest sizes.

* gemm_bias_gelu rejects 256*K*2 >= 2^32 - 16, so the largest K (a multiple
  of 8) is 8388600: A and W of 4 GiB each on one 256 x 256 tile, row offsets
  up to 2^32.  A[m, k] = r(k)/8 where k = m mod 4096 (r(k) = 1 + floor(4k/K),
  different in each quarter of K) and 0 elsewhere; W[n, k] = 1 where
  k = n mod 4096.  The product is then diagonal with exact entries
  sum_{k = m mod 4096} r(k)/8 (integers times 1/8, exact in fp32).
* M = 2^23 rows with N = 256, K = 64: C of 4 GiB.  W[n] = e_(n mod 64), so the
  pre-activation is A[m, n mod 64] + bias[n], with A[m, k] =
  ((m + k) mod 7 - 3)/4 and bias[n] = (n mod 5 - 2)/4: 35 distinct values.
* row_softmax and rmsnorm_silu on 2^24 rows of 256 (8 GiB in, 8 GiB out):
  x[r, c] = ((r + c) mod 11 - 5)/2, so row r equals row r mod 11.

The expected values are the float64 oracle's (GELU of the 35 pre-activations,
the row kernels on the 11 distinct rows), compared with the bars of the
ordinary parity tests: |y - y_ref| <= 2^-10 max(|y_ref|, 1) for the fp16 GEMM,
2^-10 |y_ref| + floor for the fp16 row kernels.
"""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_dev():
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    return torch


@pytest.fixture(scope="module")
def fa():
    from tile_level_programming_amd import fa as mod

    return mod


def _f16_bits(x):
    return np.asarray(x, dtype=np.float16).view(np.uint16)


def test_gemm_largest_k(torch_dev, fa):
    import oracle.gemm as og

    torch = torch_dev
    M = N = 256
    K = ((1 << 32) - 16) // 512 // 8 * 8
    while 256 * K * 2 >= (1 << 32) - 16:
        K -= 8
    print(f"\n[limits] gemm M={M} N={N} K={K}: building A and W (8 GiB)", flush=True)
    a = torch.zeros(M, K, dtype=torch.float16, device="cuda")
    w = torch.zeros(N, K, dtype=torch.float16, device="cuda")
    diag = np.zeros(M)
    for m in range(M):
        ks = torch.arange(m, K, 4096, device="cuda")
        r = 1 + torch.div(4 * ks, K, rounding_mode="floor")
        a[m, m::4096] = (r.to(torch.float32) / 8).to(torch.float16)
        w[m, m::4096] = 1.0
        kk = np.arange(m, K, 4096, dtype=np.int64)
        diag[m] = float((1 + (4 * kk) // K).sum()) / 8
    bias = torch.from_numpy(((np.arange(N) % 5 - 2) / 4).astype(np.float16)).cuda()
    print(f"[limits] gemm K={K}: run", flush=True)
    c = fa.linear_gelu(a, w, bias)
    torch.cuda.synchronize()
    b64 = (np.arange(N) % 5 - 2) / 4
    pre = np.diag(diag) + b64[None, :]
    ref = np.vectorize(og.gelu)(pre)
    got = c.float().double().cpu().numpy()
    err = np.abs(got - ref) - 2.0 ** -10 * np.maximum(np.abs(ref), 1.0)
    print(f"[limits] gemm K={K}: worst margin {err.max():.3e}", flush=True)
    assert np.all(np.isfinite(got)) and err.max() <= 0
    del a, w, c
    torch.cuda.empty_cache()


def test_gemm_largest_m(torch_dev, fa):
    import oracle.gemm as og

    torch = torch_dev
    M, N, K = 1 << 23, 256, 64
    print(f"\n[limits] gemm M={M} N={N} K={K}: building A (1 GiB), C is 4 GiB", flush=True)
    m_idx = torch.arange(M, device="cuda", dtype=torch.int32)[:, None]
    k_idx = torch.arange(K, device="cuda", dtype=torch.int32)[None, :]
    a = ((((m_idx + k_idx) % 7) - 3).to(torch.float32) / 4).to(torch.float16)
    del m_idx
    w = torch.zeros(N, K, dtype=torch.float16, device="cuda")
    w[torch.arange(N), torch.arange(N) % K] = 1.0
    bias = torch.from_numpy(((np.arange(N) % 5 - 2) / 4).astype(np.float16)).cuda()
    print(f"[limits] gemm M={M}: run", flush=True)
    c = fa.linear_gelu(a, w, bias)
    torch.cuda.synchronize()
    del a
    # table of the 35 pre-activations: (i - 3)/4 + (j - 2)/4, i = (m + n mod 64) mod 7, j = n mod 5
    table = np.array([[og.gelu((i - 3) / 4 + (j - 2) / 4) for j in range(5)] for i in range(7)])
    tab = torch.from_numpy(table).cuda()
    n = torch.arange(N, device="cuda")
    worst = -1.0
    step = 1 << 20
    for m0 in range(0, M, step):
        m = torch.arange(m0, m0 + step, device="cuda")[:, None]
        ref = tab[(m + (n % K)[None, :]) % 7, (n % 5)[None, :]]
        got = c[m0:m0 + step].double()
        margin = (got - ref).abs() - 2.0 ** -10 * torch.clamp(ref.abs(), min=1.0)
        worst = max(worst, margin.max().item())
    print(f"[limits] gemm M={M}: worst margin {worst:.3e}", flush=True)
    assert worst <= 0
    del c
    torch.cuda.empty_cache()


@pytest.mark.parametrize("op", ["softmax", "rmsnorm_silu"])
def test_rows_largest_r(torch_dev, fa, op):
    import oracle.rowwise as ro

    torch = torch_dev
    R, C, eps = 1 << 24, 256, 1e-6
    print(f"\n[limits] {op} R={R} C={C}: building x (8 GiB)", flush=True)
    c_idx = torch.arange(C, device="cuda", dtype=torch.int32)[None, :]
    x = torch.empty(R, C, dtype=torch.float16, device="cuda")
    step = 1 << 20
    for r0 in range(0, R, step):
        r = torch.arange(r0, r0 + step, device="cuda", dtype=torch.int32)[:, None]
        x[r0:r0 + step] = ((((r + c_idx) % 11) - 5).to(torch.float32) / 2).to(torch.float16)
    g_bits = _f16_bits((np.arange(C) % 3 + 1) * 0.5)
    g = torch.from_numpy(g_bits.view(np.int16)).view(torch.float16).cuda()
    print(f"[limits] {op} R={R}: run", flush=True)
    y = fa.softmax(x) if op == "softmax" else fa.rmsnorm_silu_rows(x, g, eps)
    torch.cuda.synchronize()
    del x
    base = _f16_bits((((np.arange(11)[:, None] + np.arange(C)[None, :]) % 11) - 5) / 2)
    ref11 = ro.softmax_rows(base, "f16") if op == "softmax" else ro.rmsnorm_silu_rows(base, g_bits, "f16", eps)
    tab = torch.from_numpy(ref11).cuda()
    floor = 2.0 ** -24 if op == "softmax" else 1e-5
    worst = -1.0
    for r0 in range(0, R, step):
        r = torch.arange(r0, r0 + step, device="cuda")
        ref = tab[r % 11]
        got = y[r0:r0 + step].double()
        margin = (got - ref).abs() - (2.0 ** -10 * ref.abs() + floor)
        worst = max(worst, margin.max().item())
    print(f"[limits] {op} R={R}: worst margin {worst:.3e}", flush=True)
    assert worst <= 0
    del y
    torch.cuda.empty_cache()

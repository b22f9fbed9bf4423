"""GPU parity of the GEMM with the fused bias + GELU epilogue (gemm_bias_gelu)
against the float64 oracle, through the C ABI.

Tolerance, from the arithmetic: the product is accumulated in fp32 and the
result rounded once to the output type, so the error is half an ulp of the
output type plus the fp32 accumulation and erff errors.  The bar is one ulp
relative to max(|c_ref|, 1): |c - c_ref| <= 2^-10 max(|c_ref|, 1) for fp16,
2^-7 max(|c_ref|, 1) for bf16.
"""

import os

import numpy as np
import pytest

import fa_inputs as fi

pytestmark = pytest.mark.gpu

REL = {"f16": 2.0 ** -10, "bf16": 2.0 ** -7}
THREADS = min(16, os.cpu_count() or 1)


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


@pytest.fixture(scope="module")
def go():
    import oracle.gemm as g

    g._load()
    return g


def to_dev(torch, bits, dtype):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.float16 if dtype == "f16" else torch.bfloat16).cuda()


def check(c, c_ref, dtype, what):
    assert np.all(np.isfinite(c)), f"{what}: non-finite output"
    err = np.abs(c - c_ref) / np.maximum(np.abs(c_ref), 1.0)
    i = np.unravel_index(np.argmax(err), err.shape)
    assert err.max() <= REL[dtype], f"{what}: error {err.max():.3e} (x ulp bar) at {i}: {c[i]} vs {c_ref[i]}"


def run(torch, fa, a, w, b, dtype, guard=4096):
    M, K = a.shape
    N = w.shape[0]
    ad, wd = to_dev(torch, a, dtype), to_dev(torch, w, dtype)
    bd = to_dev(torch, b, dtype) if b is not None else None
    tdt = ad.dtype
    buf = torch.full((guard + M * N + guard,), float("nan"), dtype=tdt, device="cuda")
    c = buf[guard:guard + M * N].view(M, N)
    st = fa.gemm_bias_gelu(ad.data_ptr(), wd.data_ptr(), 0 if bd is None else bd.data_ptr(), c.data_ptr(),
                           M, N, K, fa.FA_F16 if dtype == "f16" else fa.FA_BF16,
                           torch.cuda.current_stream().cuda_stream)
    assert st == fa.FA_OK, fa.fa_status_string(st)
    torch.cuda.synchronize()
    assert bool(torch.isnan(buf[:guard]).all()) and bool(torch.isnan(buf[guard + M * N:]).all()), "guard overwritten"
    return c.float().double().cpu().numpy()


def inputs(seed, M, N, K, dtype, bias=True):
    w = fi.GemmWorkload("t", M, N, K, dtype, seed, bias=bias)
    return fi.make_gemm_inputs(w)


SHAPES = [
    # (M, N, K, dtype, bias)
    (128, 128, 32, "f16", True),
    (128, 128, 64, "bf16", True),
    (1, 1, 8, "f16", True),
    (300, 200, 72, "f16", True),
    (129, 257, 520, "bf16", False),
    (256, 384, 1024, "f16", True),
    (1000, 130, 264, "bf16", True),
    (77, 1030, 40, "f16", True),        # N not a multiple of 4: element stores
    (513, 64, 2048, "bf16", True),
    # K slab counts (64 wide) around the six-slab unroll: 3, 4, 6, 7, 13
    (260, 300, 136, "f16", True),
    (256, 256, 256, "bf16", True),
    (200, 520, 384, "bf16", False),
    (300, 256, 392, "f16", True),
    (129, 130, 776, "bf16", True),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "m{}_n{}_k{}_{}_{}".format(*s))
def test_gemm_parity(torch_dev, fa, go, shape):
    M, N, K, dtype, bias = shape
    print(f"[gemm] {shape}", flush=True)
    a, w, b = inputs(61, M, N, K, dtype, bias)
    c = run(torch_dev, fa, a, w, b, dtype)
    check(c, go.gemm_rows(a, w, b, dtype, threads=THREADS), dtype, str(shape))


def test_gemm_zero_input_and_identity_weight(torch_dev, fa, go):
    dtype = "f16"
    K = 64
    a, _, b = inputs(62, 200, K, K, dtype)
    w = fi.f32_to_bits(np.eye(K, dtype=np.float32), dtype)
    c = run(torch_dev, fa, a, w, b, dtype)
    check(c, go.gemm_rows(a, w, b, dtype), dtype, "identity weight")
    z = np.zeros_like(a)
    cz = run(torch_dev, fa, z, w, b, dtype)
    assert np.all(cz == cz[0]), "zero input: every row is gelu(bias)"
    check(cz[:1], go.gemm_rows(z[:1], w, b, dtype), dtype, "zero input")


def test_gemm_large_values(torch_dev, fa, go):
    # un-normalised weights: pre-activations of size ~sqrt(K), where GELU is
    # the identity (positive) or 0 (negative) and the output rounding dominates
    dtype = "bf16"
    M, N, K = 256, 256, 512
    a = fi.tensor_bits(63, "a", (M, K), dtype)
    w = fi.tensor_bits(63, "w", (N, K), dtype)
    b = fi.tensor_bits(63, "bias", (N,), dtype)
    check(run(torch_dev, fa, a, w, b, dtype), go.gemm_rows(a, w, b, dtype, threads=THREADS), dtype, "large")


def test_gemm_deterministic(torch_dev, fa):
    dtype = "bf16"
    a, w, b = inputs(64, 384, 512, 640, dtype)
    c1 = run(torch_dev, fa, a, w, b, dtype)
    c2 = run(torch_dev, fa, a, w, b, dtype)
    assert np.array_equal(c1, c2)


@pytest.mark.parametrize("name", list(fi.GEMM_WORKLOADS))
def test_gemm_workload_parity(torch_dev, fa, go, name):
    # the benchmarked shapes at full size, on sampled rows the oracle
    # evaluates one by one (all columns of each): two rows at seeded offsets
    # in every 256-row block, so every 256 x 256 output tile is checked
    torch = torch_dev
    wl = fi.GEMM_WORKLOADS[name]
    print(f"[gemm] workload {name}", flush=True)
    a, w, b = fi.make_gemm_inputs(wl)
    ad, wd = to_dev(torch, a, wl.dtype), to_dev(torch, w, wl.dtype)
    bd = to_dev(torch, b, wl.dtype) if b is not None else None
    c = fa.linear_gelu(ad, wd, bd)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    blocks = np.arange(0, wl.M, 256)
    rows = np.concatenate([[0, 127, 128, wl.M - 1], blocks + rng.integers(0, 256, blocks.size),
                           blocks + rng.integers(0, 256, blocks.size)])
    rows = np.unique(rows[rows < wl.M])
    cs = c[torch.from_numpy(rows).cuda()].float().double().cpu().numpy()
    check(cs, go.gemm_rows(a, w, b, wl.dtype, rows=rows, threads=THREADS), wl.dtype, name)
    assert bool(torch.isfinite(c.float()).all())

"""GPU parity of the HIP attention forward pass against the float64 oracle.

All calls go through the C ABI (via the ctypes binding).  Inputs are the
seeded bit patterns of ``fa_inputs``; the oracle consumes the same bits.

Tolerances (the acceptance bar of the port): max |O - O_ref| <= 5e-3 for
fp16 and <= 2e-2 for bf16; |lse - lse_ref| / max(|lse_ref|, 1) <= 1e-3.  The
guarded denominator keeps the lse bound meaningful for rows whose lse is near
zero (e.g. the first causal row, whose lse is a single logit).
"""

import math
import os

import numpy as np
import pytest

import fa_inputs as fi

pytestmark = pytest.mark.gpu

TOL_O = {"f16": 5e-3, "bf16": 2e-2}
TOL_LSE = 1e-3
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


def to_dev(torch, bits, dtype):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    t = t.view(torch.float16 if dtype == "f16" else torch.bfloat16)
    return t.cuda()


def to_f64(torch, t):
    return t.float().double().cpu().numpy()


def run_gpu(torch, fa, q, k, v, dtype, scale, causal, prefill=float("nan")):
    qd, kd, vd = (to_dev(torch, x, dtype) for x in (q, k, v))
    o = torch.full_like(qd, prefill)
    lse = torch.full(qd.shape[:3], prefill, dtype=torch.float32, device=qd.device)
    fa.fwd(qd, kd, vd, causal=causal, scale=scale, out=o, lse=lse)
    torch.cuda.synchronize()
    return o, lse


def check(o_gpu, lse_gpu, o_ref, lse_ref, dtype, what=""):
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite O"
    assert np.all(np.isfinite(lse_gpu)), f"{what}: non-finite lse"
    err_o = np.abs(o_gpu - o_ref)
    i = np.unravel_index(np.argmax(err_o), err_o.shape)
    assert err_o.max() <= TOL_O[dtype], f"{what}: max |dO| {err_o.max():.3e} at {i}"
    err_l = np.abs(lse_gpu - lse_ref) / np.maximum(np.abs(lse_ref), 1.0)
    j = np.unravel_index(np.argmax(err_l), err_l.shape)
    assert err_l.max() <= TOL_LSE, f"{what}: max lse err {err_l.max():.3e} at {j}"
    return float(err_o.max()), float(err_l.max())


def full_check(torch, fa, oracle_mod, q, k, v, dtype, scale, causal, what=""):
    o, lse = run_gpu(torch, fa, q, k, v, dtype, scale, causal)
    o_ref, lse_ref = oracle_mod.attention(q, k, v, dtype, scale, causal, threads=THREADS)
    return check(to_f64(torch, o), lse.double().cpu().numpy(), o_ref, lse_ref, dtype, what)


# --- the five measured shapes (six runs) -------------------------------------


@pytest.mark.parametrize("name", list(fi.WORKLOADS))
def test_workload_parity(torch_dev, fa, oracle_mod, name):
    # every row of every workload against the threaded oracle (the largest,
    # B1 H32 S16384 D128 causal, is about 3e12 float64 operations: well under
    # a minute on 16 host threads)
    torch = torch_dev
    w = fi.WORKLOADS[name]
    print(f"[parity] {name}: all {w.B * w.H * w.Sq} rows", flush=True)
    q, k, v = fi.make_inputs(w)
    o, lse = run_gpu(torch, fa, q, k, v, w.dtype, w.scale, w.causal)
    o_gpu, l_gpu = to_f64(torch, o), lse.double().cpu().numpy()
    del o, lse
    o_ref, l_ref = oracle_mod.attention(q, k, v, w.dtype, w.scale, w.causal, threads=THREADS)
    err_o, err_l = check(o_gpu, l_gpu, o_ref, l_ref, w.dtype, name)
    raw = float(np.abs(l_gpu - l_ref).max())
    rel_raw = float((np.abs(l_gpu - l_ref) / np.abs(l_ref)).max())
    small = int((np.abs(l_ref) < 1).sum())
    print(f"[parity] {name}: max|dO| {err_o:.3e} (bar {TOL_O[w.dtype]:.0e}); lse error guarded {err_l:.3e}, "
          f"unguarded relative {rel_raw:.3e}, absolute {raw:.3e}; rows with |lse_ref| < 1: {small}", flush=True)


# --- ragged and odd shapes ---------------------------------------------------

ODD = [
    # (B, H, Sq, Sk, D)
    (1, 1, 1, 1, 64), (1, 2, 17, 17, 64), (2, 1, 77, 200, 128), (1, 1, 200, 77, 64),
    (1, 3, 1000, 1000, 128), (1, 1, 129, 1, 64), (1, 1, 1, 1000, 128), (2, 2, 255, 257, 64),
    (1, 1, 64, 64, 128), (1, 1, 1000, 17, 128),
]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", ODD)
def test_odd_shapes(torch_dev, fa, oracle_mod, shape, causal, dtype):
    B, H, Sq, Sk, D = shape
    seed = 100 + Sq + 7 * Sk
    q = fi.tensor_bits(seed, "q", (B, H, Sq, D), dtype)
    k = fi.tensor_bits(seed, "k", (B, H, Sk, D), dtype)
    v = fi.tensor_bits(seed, "v", (B, H, Sk, D), dtype)
    full_check(torch_dev, fa, oracle_mod, q, k, v, dtype, 1.0 / math.sqrt(D), causal, f"{shape} {causal} {dtype}")


# Many heads with short, ragged sequences: grids of hundreds of work-groups
# whose query and key ends fall inside tiles.
WIDE = [
    # (B, H, Sq, Sk, D)
    (2, 128, 200, 333, 64), (1, 256, 77, 77, 128), (4, 64, 300, 129, 128), (1, 256, 256, 1000, 64),
    (1, 256, 257, 31, 64),
    # D=64 launches of more than 512 work-groups take the 32-key tiles, the
    # smaller ones above the 64-key tiles
    (2, 160, 300, 333, 64), (1, 300, 200, 515, 64),
]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", WIDE)
def test_wide_grid_shapes(torch_dev, fa, oracle_mod, shape, causal, dtype):
    B, H, Sq, Sk, D = shape
    seed = 300 + Sq + 3 * Sk + D
    q = fi.tensor_bits(seed, "q", (B, H, Sq, D), dtype)
    k = fi.tensor_bits(seed, "k", (B, H, Sk, D), dtype)
    v = fi.tensor_bits(seed, "v", (B, H, Sk, D), dtype)
    full_check(torch_dev, fa, oracle_mod, q, k, v, dtype, 1.0 / math.sqrt(D), causal, f"{shape} {causal} {dtype}")


# Shapes on both sides of the launch choices, which depend on the number of
# 128-query blocks B*H*ceil(Sq/128): up to 128 run as two key groups of two
# waves (64 queries per work-group), up to 512 (D=64) with 64-key tiles, beyond
# with 32-key tiles.  The keys end inside a tile.
BOUNDARY = [
    # (B, H, Sq, Sk, D, dtype)        blocks
    (1, 16, 1024, 1061, 64, "f16"),   # 128
    (1, 43, 384, 421, 64, "f16"),     # 129
    (2, 32, 1024, 1061, 64, "f16"),   # 512
    (1, 171, 384, 421, 64, "f16"),    # 513
    (1, 16, 1024, 1061, 128, "bf16"),  # 128
    (1, 43, 384, 421, 128, "bf16"),   # 129
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", BOUNDARY)
def test_launch_boundary_shapes(torch_dev, fa, oracle_mod, shape, causal):
    B, H, Sq, Sk, D, dtype = shape
    seed = 500 + H + Sq
    q = fi.tensor_bits(seed, "q", (B, H, Sq, D), dtype)
    k = fi.tensor_bits(seed, "k", (B, H, Sk, D), dtype)
    v = fi.tensor_bits(seed, "v", (B, H, Sk, D), dtype)
    full_check(torch_dev, fa, oracle_mod, q, k, v, dtype, 1.0 / math.sqrt(D), causal, f"{shape} {causal}")


@pytest.mark.parametrize("scale", [-0.2, 0.0, 1.0, 3.0])
@pytest.mark.parametrize("causal", [False, True])
def test_scales(torch_dev, fa, oracle_mod, scale, causal):
    dtype = "f16"
    q = fi.tensor_bits(21, "q", (1, 2, 300, 64), dtype)
    k = fi.tensor_bits(21, "k", (1, 2, 300, 64), dtype)
    v = fi.tensor_bits(21, "v", (1, 2, 300, 64), dtype)
    full_check(torch_dev, fa, oracle_mod, q, k, v, dtype, scale, causal, f"scale {scale}")


def test_large_logits_rescaling(torch_dev, fa, oracle_mod):
    # sigma 4 inputs at D=128: logits with spread ~ 16*sqrt(128)/sqrt(128) ... large
    # running-max jumps in every tile
    dtype = "bf16"
    q = fi.tensor_bits(22, "q", (1, 2, 600, 128), dtype, 4.0)
    k = fi.tensor_bits(22, "k", (1, 2, 600, 128), dtype, 4.0)
    v = fi.tensor_bits(22, "v", (1, 2, 600, 128), dtype)
    for causal in (False, True):
        full_check(torch_dev, fa, oracle_mod, q, k, v, dtype, 1.0 / math.sqrt(128), causal, "sigma4")


def _bits_to_f32(bits, dtype):
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float32)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


@pytest.mark.parametrize("D,dtype,H", [(64, "f16", 2), (128, "bf16", 2), (64, "bf16", 2), (128, "f16", 2),
                                       (64, "f16", 192), (64, "bf16", 192)])
@pytest.mark.parametrize("causal", [False, True])
def test_rising_logits(torch_dev, fa, oracle_mod, D, dtype, H, causal):
    # keys scaled up along the sequence: each row's maximum keeps growing,
    # so the kernel's reference has to move many times, in the branch-free
    # steps and in the masked tail, both before and after a tile's products.
    # At D=64, H=2 runs the 64-key tiles and H=192 (576 work-groups) the
    # 32-key tiles.  The dominant keys of these nearly one-hot rows sit in
    # the masked tail, whose P (up to the sum bound above the reference) bf16
    # rounds by up to 2^-9: the normaliser must sum the same rounded P as the
    # P.V product there too, or O is scaled by the rounding (bf16, 192 heads:
    # max |dO| 2.05e-2 with fp32 sums of the unrounded P on those steps).
    Sq, Sk = 300, 2000
    q = fi.tensor_bits(24, "q", (1, H, Sq, D), dtype, 2.0)
    k0 = _bits_to_f32(fi.tensor_bits(24, "k", (1, H, Sk, D), dtype), dtype)
    ramp = (0.25 + 6.0 * np.arange(Sk, dtype=np.float32) / Sk)[None, None, :, None]
    k = fi.f32_to_bits(k0 * ramp, dtype)
    v = fi.tensor_bits(24, "v", (1, H, Sk, D), dtype)
    err_o, err_l = full_check(torch_dev, fa, oracle_mod, q, k, v, dtype, 1.0 / math.sqrt(D), causal,
                              f"rising {D} {dtype}")
    print(f"[rising] D={D} {dtype} H={H} causal={causal}: max|dO| {err_o:.4e} lse err {err_l:.3e}", flush=True)


@pytest.mark.parametrize("D,dtype,H", [(64, "f16", 2), (128, "bf16", 2), (64, "f16", 180)])
@pytest.mark.parametrize("causal", [False, True])
def test_nan_query_rows_stay_in_their_rows(torch_dev, fa, oracle_mod, D, dtype, H, causal):
    # A NaN in a query row makes that row's scores, O and lse NaN and must
    # leave every other row exact.  Rows 16 and 140 pair with rows 0 and 124
    # in the matrix-unit row sums (query n and n+16 of a wave share a column
    # there), rows 5 and 21 are such a pair both poisoned.
    torch = torch_dev
    Sq, Sk = 300, 1500
    q = fi.tensor_bits(26, "q", (1, H, Sq, D), dtype)
    k = fi.tensor_bits(26, "k", (1, H, Sk, D), dtype)
    v = fi.tensor_bits(26, "v", (1, H, Sk, D), dtype)
    bad = [5, 16, 21, 140]
    qn = q.copy()
    qn[0, 0, bad, 3] = 0x7E00 if dtype == "f16" else 0x7FC0
    o, lse = run_gpu(torch, fa, qn, k, v, dtype, 1.0 / math.sqrt(D), causal)
    o, lse = to_f64(torch, o), lse.double().cpu().numpy()
    assert np.all(np.isnan(o[0, 0, bad])) and np.all(np.isnan(lse[0, 0, bad]))
    good = np.ones((1, H, Sq), bool)
    good[0, 0, bad] = False
    o_ref, lse_ref = oracle_mod.attention(q, k, v, dtype, 1.0 / math.sqrt(D), causal, threads=THREADS)
    check(o[good], lse[good], o_ref[good], lse_ref[good], dtype, f"nan rows {D} {dtype}")


# --- properties checkable without the oracle ---------------------------------


@pytest.mark.parametrize("causal", [False, True])
def test_zero_q_gives_prefix_mean(torch_dev, fa, causal):
    torch = torch_dev
    dtype = "f16"
    Sq = Sk = 333
    q = np.zeros((1, 1, Sq, 64), np.uint16)
    k = fi.tensor_bits(23, "k", (1, 1, Sk, 64), dtype)
    v = fi.tensor_bits(23, "v", (1, 1, Sk, 64), dtype)
    o, lse = run_gpu(torch, fa, q, k, v, dtype, 0.125, causal)
    vv = to_f64(torch, to_dev(torch, v, dtype))[0, 0]
    n = np.arange(1, Sq + 1) if causal else np.full(Sq, Sk)
    mean = np.cumsum(vv, axis=0) / np.arange(1, Sk + 1)[:, None] if causal else np.broadcast_to(vv.mean(0), (Sq, 64))
    np.testing.assert_allclose(to_f64(torch, o)[0, 0], mean, atol=TOL_O[dtype])
    np.testing.assert_allclose(lse.double().cpu().numpy()[0, 0], np.log(n), rtol=1e-5, atol=1e-5)


def test_constant_v(torch_dev, fa):
    torch = torch_dev
    for dtype in ("f16", "bf16"):
        q = fi.tensor_bits(24, "q", (1, 2, 257, 128), dtype, 2.0)
        k = fi.tensor_bits(24, "k", (1, 2, 257, 128), dtype, 2.0)
        row = fi.tensor_bits(24, "v", (1, 2, 1, 128), dtype)
        v = np.ascontiguousarray(np.broadcast_to(row, (1, 2, 257, 128)))
        o, _ = run_gpu(torch, fa, q, k, v, dtype, 0.1, True)
        want = to_f64(torch, to_dev(torch, row, dtype))
        np.testing.assert_allclose(to_f64(torch, o), np.broadcast_to(want, (1, 2, 257, 128)),
                                   atol=TOL_O[dtype])


def test_outputs_fully_written_and_guards_intact(torch_dev, fa):
    torch = torch_dev
    dtype = "f16"
    B, H, Sq, Sk, D = 1, 3, 190, 70, 64
    q = to_dev(torch, fi.tensor_bits(25, "q", (B, H, Sq, D), dtype), dtype)
    k = to_dev(torch, fi.tensor_bits(25, "k", (B, H, Sk, D), dtype), dtype)
    v = to_dev(torch, fi.tensor_bits(25, "v", (B, H, Sk, D), dtype), dtype)
    n_o = B * H * Sq * D
    n_l = B * H * Sq
    guard = 4096
    ob = torch.full((guard + n_o + guard,), float("nan"), dtype=torch.float16, device="cuda")
    lb = torch.full((guard + n_l + guard,), float("nan"), dtype=torch.float32, device="cuda")
    ob[:guard] = 7.0
    ob[-guard:] = 7.0
    lb[:guard] = 7.0
    lb[-guard:] = 7.0
    o = ob[guard:guard + n_o].view(B, H, Sq, D)
    lse = lb[guard:guard + n_l].view(B, H, Sq)
    for causal in (False, True):
        fa.fwd(q, k, v, causal=causal, out=o, lse=lse)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
        assert bool((ob[:guard] == 7).all()) and bool((ob[-guard:] == 7).all())
        assert bool((lb[:guard] == 7).all()) and bool((lb[-guard:] == 7).all())


def test_deterministic(torch_dev, fa):
    torch = torch_dev
    w = fi.WORKLOADS["causal_b2h8_s1024_d64_f16"]
    q, k, v = (to_dev(torch, x, w.dtype) for x in fi.make_inputs(w))
    o1, l1 = fa.fwd(q, k, v, causal=True)
    o2, l2 = fa.fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))


def test_side_stream(torch_dev, fa, oracle_mod):
    torch = torch_dev
    dtype = "bf16"
    q = fi.tensor_bits(26, "q", (1, 2, 256, 128), dtype)
    k = fi.tensor_bits(26, "k", (1, 2, 256, 128), dtype)
    v = fi.tensor_bits(26, "v", (1, 2, 256, 128), dtype)
    qd, kd, vd = (to_dev(torch, x, dtype) for x in (q, k, v))
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o, lse = fa.fwd(qd, kd, vd, causal=False)
    s.synchronize()
    o_ref, l_ref = oracle_mod.attention(q, k, v, dtype, 1 / math.sqrt(128), False, threads=THREADS)
    check(to_f64(torch, o), lse.double().cpu().numpy(), o_ref, l_ref, dtype, "side stream")


def test_device_errors_are_host_errors(torch_dev, fa):
    torch = torch_dev
    q = torch.zeros(1, 1, 8, 64, dtype=torch.float16, device="cuda")
    with pytest.raises(fa.FaError):
        fa.fwd(q, q, q, out=q)  # output aliases the input
    with pytest.raises(fa.FaError):
        fa.fwd(torch.zeros(1, 1, 8, 96, dtype=torch.float16, device="cuda"),
               torch.zeros(1, 1, 8, 96, dtype=torch.float16, device="cuda"),
               torch.zeros(1, 1, 8, 96, dtype=torch.float16, device="cuda"))


def test_bad_outputs_rejected_before_launch(torch_dev, fa):
    torch = torch_dev
    q = torch.zeros(1, 2, 8, 64, dtype=torch.float16, device="cuda")
    with pytest.raises(ValueError):
        fa.fwd(q, q, q, out=torch.empty(1, 2, 7, 64, dtype=torch.float16, device="cuda"))
    with pytest.raises(TypeError):
        fa.fwd(q, q, q, out=torch.empty(1, 2, 8, 64, dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        fa.fwd(q, q, q, out=torch.empty(1, 2, 64, 8, dtype=torch.float16, device="cuda").transpose(2, 3))
    with pytest.raises(TypeError):
        fa.fwd(q, q, q, lse=torch.empty(1, 2, 8, dtype=torch.float16, device="cuda"))
    with pytest.raises(ValueError):
        fa.fwd(q, q, q, lse=torch.empty(1, 2, 8, dtype=torch.float32))
    with pytest.raises(ValueError):
        fa.fwd_split(q, q, q, lse=torch.empty(2, 8, dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError):
        fa.linear_gelu(torch.zeros(4, 8, dtype=torch.float16, device="cuda"),
                       torch.zeros(6, 8, dtype=torch.float16, device="cuda"),
                       out=torch.empty(4, 5, dtype=torch.float16, device="cuda"))
    with pytest.raises(ValueError):
        fa.softmax(torch.zeros(4, 8, dtype=torch.float16, device="cuda"),
                   out=torch.empty(4, 8, dtype=torch.float16))

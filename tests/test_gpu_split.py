"""GPU parity of the key-split forward pass (fa_fwd_split) and of the
log-sum-exp merge (fa_lse_merge) against the float64 oracle.

The split result is checked against the unsplit oracle (it must be the same
attention), the workspace partials against the oracle over each key range,
and the merge on its own against the oracle's merge.  Tolerances as for
fa_fwd: max |O - O_ref| <= 5e-3 (fp16), 2e-2 (bf16); lse relative 1e-3.
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
    return t.view(torch.float16 if dtype == "f16" else torch.bfloat16).cuda()


def check(o, lse, o_ref, lse_ref, dtype, what):
    assert np.all(np.isfinite(o)), f"{what}: non-finite O"
    err_o = np.abs(o - o_ref)
    assert err_o.max() <= TOL_O[dtype], f"{what}: max |dO| {err_o.max():.3e} at {np.unravel_index(err_o.argmax(), err_o.shape)}"
    err_l = np.abs(lse - lse_ref) / np.maximum(np.abs(lse_ref), 1.0)
    assert err_l.max() <= TOL_LSE, f"{what}: max lse err {err_l.max():.3e}"
    return float(err_o.max()), float(err_l.max())


def inputs(seed, B, H, Sq, Sk, D, dtype, sigma=1.0):
    q = fi.tensor_bits(seed, "q", (B, H, Sq, D), dtype, sigma)
    k = fi.tensor_bits(seed, "k", (B, H, Sk, D), dtype, sigma)
    v = fi.tensor_bits(seed, "v", (B, H, Sk, D), dtype)
    return q, k, v


def run_split(torch, fa, q, k, v, dtype, causal, n_split, scale=None):
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    qd, kd, vd = (to_dev(torch, x, dtype) for x in (q, k, v))
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((B, H, Sq), float("nan"), dtype=torch.float32, device="cuda")
    need = fa.split_workspace_size(B, H, Sq, Sk, D, n_split)
    guard = 4096
    ws = torch.full((guard + need + guard,), 0x7F, dtype=torch.uint8, device="cuda")
    wsv = ws[guard:guard + need]
    fa.fwd_split(qd, kd, vd, causal=causal, scale=scale, n_split=n_split, out=o, lse=lse, workspace=wsv)
    torch.cuda.synchronize()
    assert bool((ws[:guard] == 0x7F).all()) and bool((ws[guard + need:] == 0x7F).all()), "workspace guard overwritten"
    return o, lse, wsv


SHAPES = [
    # (B, H, Sq, Sk, D, dtype, causal, n_split)
    (2, 4, 1, 5000, 64, "f16", False, 0),
    (2, 4, 1, 5000, 64, "f16", False, 1),
    (1, 8, 4, 8229, 128, "bf16", False, 3),
    (1, 8, 4, 8229, 128, "bf16", True, 0),
    (1, 2, 300, 3000, 64, "f16", True, 5),
    (1, 2, 300, 3000, 128, "f16", False, 0),
    (1, 3, 200, 100, 64, "bf16", True, 7),
    (3, 2, 17, 2049, 64, "bf16", True, 0),
    (1, 1, 129, 777, 128, "f16", True, 4),
    # D=64 launches of more than 512 work-groups (32-key tiles)
    (4, 64, 16, 9000, 64, "f16", False, 0),
    (2, 128, 300, 2000, 64, "bf16", True, 3),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "b{}h{}_sq{}_sk{}_d{}_{}_{}_n{}".format(*s))
def test_split_parity(torch_dev, fa, oracle_mod, shape):
    torch = torch_dev
    B, H, Sq, Sk, D, dtype, causal, n_split = shape
    print(f"[split] {shape}", flush=True)
    q, k, v = inputs(41, B, H, Sq, Sk, D, dtype)
    o, lse, _ = run_split(torch, fa, q, k, v, dtype, causal, n_split)
    o_ref, lse_ref = oracle_mod.attention(q, k, v, dtype, 1.0 / math.sqrt(D), causal, threads=THREADS)
    check(o.float().double().cpu().numpy(), lse.double().cpu().numpy(), o_ref, lse_ref, dtype, str(shape))


@pytest.mark.parametrize("causal", [False, True])
def test_split_partials_are_key_range_attention(torch_dev, fa, oracle_mod, causal):
    # the workspace holds, per key range, O normalised over the range and its
    # lse; rows that see no key of a range hold 0 and -inf
    torch = torch_dev
    B, H, Sq, Sk, D, dtype = 1, 2, 260, 1000, 64, "f16"
    q, k, v = inputs(42, B, H, Sq, Sk, D, dtype, 1.5)
    n = fa.split_count(B, H, Sq, Sk, 4)
    chunk = 256  # ceil(1000 / 4) = 250, rounded up to a multiple of 64
    assert n == 4
    _, _, ws = run_split(torch, fa, q, k, v, dtype, causal, 4)
    rows = B * H * Sq
    flat = ws.view(torch.float32)
    po = flat[:n * rows * D].view(n, rows, D).double().cpu().numpy()
    pl = flat[n * rows * D:n * rows * (D + 1)].view(n, rows).double().cpu().numpy()
    for g in range(n):
        a, b = g * chunk, min(Sk, (g + 1) * chunk)
        o_ref, l_ref = oracle_mod.attention_rows(q, k, v, dtype, 0.125, causal, key_range=(a, b), threads=THREADS)
        empty = np.isneginf(l_ref)
        assert np.array_equal(np.isneginf(pl[g]), empty), f"range {g}: empty rows differ"
        assert np.all(po[g][empty] == 0.0)
        full = ~empty
        if full.any():
            check(po[g][full], pl[g][full], o_ref[full], l_ref[full], dtype, f"range {g}")


@pytest.mark.parametrize("dtype,D", [("f16", 64), ("bf16", 128)])
def test_lse_merge_parity(torch_dev, fa, oracle_mod, dtype, D):
    torch = torch_dev
    rng = np.random.default_rng(7)
    G, R = 6, 1000
    op = rng.normal(size=(G, R, D))
    lp = rng.normal(size=(G, R)) * 20.0
    empty = rng.random((G, R)) < 0.3
    lp[empty] = -np.inf
    op[empty] = 0.0
    lp[:, 5] = -np.inf  # a row with only empty parts
    op[:, 5] = 0.0
    opt = torch.from_numpy(op.astype(np.float32)).cuda()
    lpt = torch.from_numpy(lp.astype(np.float32)).cuda()
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    o, lse = fa.lse_merge(opt, lpt, tdt)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle_mod.merge(op.astype(np.float32).astype(np.float64), lp.astype(np.float32).astype(np.float64))
    o, lse = o.float().double().cpu().numpy(), lse.double().cpu().numpy()
    assert lse[5] == -np.inf and np.all(o[5] == 0.0)
    ok = np.isfinite(l_ref)
    check(o[ok], lse[ok], o_ref[ok], l_ref[ok], dtype, "merge")


def test_split_deterministic_and_matches_unsplit(torch_dev, fa, oracle_mod):
    torch = torch_dev
    B, H, Sq, Sk, D, dtype = 1, 4, 64, 4096, 128, "bf16"
    q, k, v = inputs(43, B, H, Sq, Sk, D, dtype)
    o1, l1, _ = run_split(torch, fa, q, k, v, dtype, True, 0)
    o2, l2, _ = run_split(torch, fa, q, k, v, dtype, True, 0)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    qd, kd, vd = (to_dev(torch, x, dtype) for x in (q, k, v))
    o3, l3 = fa.fwd(qd, kd, vd, causal=True)
    torch.cuda.synchronize()
    assert (o1.float() - o3.float()).abs().max().item() <= TOL_O[dtype]
    assert ((l1 - l3).abs() / l3.abs().clamp(min=1.0)).max().item() <= TOL_LSE


@pytest.mark.parametrize("name", list(fi.DECODE_WORKLOADS))
def test_decode_workload_parity(torch_dev, fa, oracle_mod, name):
    # the benchmarked decode shapes, at full size and in the launch
    # configuration the benchmark times (automatic range count), every row
    # against the oracle
    torch = torch_dev
    w = fi.DECODE_WORKLOADS[name]
    print(f"[split] workload {name}", flush=True)
    q, k, v = fi.make_inputs(w)
    tdt = torch.float16 if w.dtype == "f16" else torch.bfloat16
    qd, kd, vd = (torch.from_numpy(x.view(np.int16)).view(tdt).cuda() for x in (q, k, v))
    o, lse = fa.fwd_split(qd, kd, vd, causal=w.causal, scale=w.scale, n_split=0)
    torch.cuda.synchronize()
    o_s = o.view(-1, w.D).double().cpu().numpy()
    l_s = lse.view(-1).double().cpu().numpy()
    o_ref, l_ref = oracle_mod.attention_rows(q, k, v, w.dtype, w.scale, w.causal, None, threads=THREADS)
    err_o, err_l = check(o_s, l_s, o_ref, l_ref, w.dtype, name)
    print(f"[split] {name}: all {o_s.shape[0]} rows, max|dO| {err_o:.3e}, lse error {err_l:.3e}", flush=True)
    assert bool(torch.isfinite(o.float()).all()) and bool(torch.isfinite(lse).all())

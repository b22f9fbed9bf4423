"""Attention at the largest key and query counts the library accepts, on one head.

``fa_fwd`` rejects Sk * D >= 2^31, so the largest inputs are Sk = 2^24 - 1 at
D = 128 and Sk = 2^25 - 1 at D = 64: K and V of 4 GiB each, byte offsets far
past 2^31.  The inputs are built so that the exact result has a closed form
(no oracle run over 2^24 keys is needed): every query is q = a*e_0 with
a = 48 and scale = 0.125, every key k_j = e_0 for j >= j1 and 0 before, so a
row's scores are 6 on the last keys and 0 on the others.  With the weights
of the two levels, Z = j1 + (Sk - j1) e^6, the output is
O_d = (sum_{j<j1} v_jd + e^6 sum_{j>=j1} v_jd) / Z and lse = ln Z (the
scaled-dot-product softmax written out for two score levels).  V is
v_jd = floor(4j/Sk) * w_d with w_d = (d mod 4) - 1.5: exact in fp16 and bf16,
different in each quarter of the keys, so dropped or repeated key ranges
change O.  The tile sum of P at the level change passes the kernel's bound,
so the running reference moves at an offset of gigabytes as well.

The query-count test takes Sq = 2^24 - 1 at D = 128 (Q and O of 4 GiB) with 100
keys on the same two score levels, against explicit float64 softmaxes over at
most 100 keys.
"""

import math

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

TOL_O = {"f16": 5e-3, "bf16": 2e-2}
TOL_LSE = 1e-3


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


def _sum_s(a, b, Sk):
    """sum of floor(4j/Sk) over integer j in [a, b), exactly."""
    tot = 0
    for t in range(4):
        lo = (t * Sk + 3) // 4          # first j with floor(4j/Sk) >= t
        hi = ((t + 1) * Sk + 3) // 4
        tot += t * max(0, min(b, hi) - max(a, lo))
    return tot


def _expected(Sk, D, j1):
    w = (np.arange(D) % 4) - 1.5
    e6 = math.exp(6.0)
    z = j1 + (Sk - j1) * e6
    o = (_sum_s(0, j1, Sk) + e6 * _sum_s(j1, Sk, Sk)) * w / z
    return o, math.log(z)


@pytest.mark.parametrize("D,dtype", [(128, "f16"), (64, "bf16")])
def test_largest_key_count(torch_dev, fa, D, dtype):
    torch = torch_dev
    Sk = (1 << 31) // D - 1
    Sq = 130  # two query blocks, the second ragged
    j1 = 3 * Sk // 4 + 7
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    print(f"\n[limits] D={D} {dtype} Sk={Sk}: building K and V ({2 * Sk * D * 2 / 2**30:.1f} GiB)", flush=True)
    q = torch.zeros(1, 1, Sq, D, dtype=tdt, device="cuda")
    q[0, 0, :, 0] = 48.0
    k = torch.zeros(1, 1, Sk, D, dtype=tdt, device="cuda")
    k[0, 0, j1:, 0] = 1.0
    v = torch.empty(1, 1, Sk, D, dtype=tdt, device="cuda")
    w = (torch.arange(D, device="cuda") % 4).to(torch.float32) - 1.5
    step = 1 << 20
    for j0 in range(0, Sk, step):
        j = torch.arange(j0, min(Sk, j0 + step), device="cuda", dtype=torch.int64)
        s = torch.div(4 * j, Sk, rounding_mode="floor").to(torch.float32)
        v[0, 0, j0:j0 + j.numel()] = (s[:, None] * w[None, :]).to(tdt)
    torch.cuda.synchronize()
    o_ref, lse_ref = _expected(Sk, D, j1)

    for how in ("fwd", "fwd_split"):
        print(f"[limits] D={D} {dtype} Sk={Sk}: {how}", flush=True)
        if how == "fwd":
            o, lse = fa.fwd(q, k, v, causal=False, scale=0.125)
        else:
            o, lse = fa.fwd_split(q, k, v, causal=False, scale=0.125)
        torch.cuda.synchronize()
        o = o.float().double().cpu().numpy()[0, 0]
        lse = lse.double().cpu().numpy()[0, 0]
        assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), how
        err_o = np.abs(o - o_ref[None, :]).max()
        err_l = (np.abs(lse - lse_ref) / max(abs(lse_ref), 1.0)).max()
        print(f"[limits] {how}: max |dO| {err_o:.2e}, lse rel {err_l:.2e}", flush=True)
        assert err_o <= TOL_O[dtype], f"{how}: max |dO| {err_o:.3e}"
        assert err_l <= TOL_LSE, f"{how}: lse error {err_l:.3e}"
    del q, k, v
    torch.cuda.empty_cache()


def _softmax_rows(q0, k0, v, scale, nkeys):
    """Explicit float64 softmax(scale * q0 * k0_j) . v over the first nkeys keys."""
    s = scale * q0 * k0[:nkeys]
    p = np.exp(s - s.max())
    return (p @ v[:nkeys]) / p.sum(), s.max() + math.log(p.sum())


@pytest.mark.parametrize("causal", [False, True])
def test_largest_query_count(torch_dev, fa, causal):
    # Sq * D < 2^31 at D = 128: Q and O of 4 GiB, 131072 work-groups, O and
    # lse offsets past 2^31; 100 keys, the last 30 on the higher score level.
    # Causal rows i < 99 see the keys 0..i, the rest see all 100.
    torch = torch_dev
    D, dtype, Sk = 128, "f16", 100
    Sq = (1 << 31) // D - 1
    j1 = 70
    print(f"\n[limits] D={D} {dtype} Sq={Sq} Sk={Sk} causal={causal}: building Q (4 GiB)", flush=True)
    q = torch.zeros(1, 1, Sq, D, dtype=torch.float16, device="cuda")
    q[0, 0, :, 0] = 48.0
    k0 = np.zeros(Sk)
    k0[j1:] = 1.0
    vh = (((np.arange(Sk) % 7) - 3)[:, None] * ((np.arange(D) % 4) - 1.5)[None, :]).astype(np.float16)
    k = torch.zeros(1, 1, Sk, D, dtype=torch.float16, device="cuda")
    k[0, 0, :, 0] = torch.from_numpy(k0.astype(np.float16)).cuda()
    v = torch.from_numpy(vh).cuda()[None, None].contiguous()
    vd = vh.astype(np.float64)
    print(f"[limits] Sq={Sq} causal={causal}: fwd", flush=True)
    o, lse = fa.fwd(q, k, v, causal=causal, scale=0.125)
    torch.cuda.synchronize()
    del q
    o_all, lse_all = _softmax_rows(48.0, k0, vd, 0.125, Sk)
    lse_h = lse.double().cpu().numpy()[0, 0]
    first = Sk - 1 if causal else 0  # rows from here on see all the keys
    ref = torch.from_numpy(o_all).to(torch.float32).cuda()[None, :]
    err_o = 0.0
    step = 1 << 20
    for i0 in range(first, Sq, step):
        blk = o[0, 0, i0:min(Sq, i0 + step)].float()
        err_o = max(err_o, (blk - ref).abs().max().item())
    err_l = np.abs(lse_h[first:] - lse_all).max() / max(abs(lse_all), 1.0)
    for i in range(first):  # causal prefixes
        o_i, l_i = _softmax_rows(48.0, k0, vd, 0.125, i + 1)
        err_o = max(err_o, float(np.abs(o[0, 0, i].double().cpu().numpy() - o_i).max()))
        err_l = max(err_l, abs(lse_h[i] - l_i) / max(abs(l_i), 1.0))
    print(f"[limits] Sq={Sq} causal={causal}: max |dO| {err_o:.2e}, lse rel {err_l:.2e}", flush=True)
    assert np.all(np.isfinite(lse_h))
    assert err_o <= TOL_O[dtype], f"max |dO| {err_o:.3e}"
    assert err_l <= TOL_LSE, f"lse error {err_l:.3e}"
    del o, lse, k, v
    torch.cuda.empty_cache()

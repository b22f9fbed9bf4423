"""The allocation-free key split (fa_fwd_split_noalloc) against the
allocating one (fa_fwd_split), through the C ABI: two calls in a row, the
second with a smaller input, each bit-identical to fa_fwd_split with the same
range count and within the attention bars of the float64 oracle."""

import math
import os

import numpy as np
import pytest

import fa_inputs as fi

pytestmark = pytest.mark.gpu

TOL_O = {"f16": 5e-3, "bf16": 2e-2}
TOL_LSE = 1e-3
THREADS = min(16, os.cpu_count() or 1)

# (B, H, Sq, Sk, D, dtype, causal, n_split): the second is the smaller call
CALLS = [(2, 4, 20, 5000, 128, "bf16", False, 0), (1, 2, 3, 700, 64, "f16", True, 3)]


def test_noalloc_matches_split_on_two_calls(oracle_mod):
    import torch

    from tile_level_programming_amd import fa

    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    stream = torch.cuda.current_stream().cuda_stream
    for i, (B, H, Sq, Sk, D, dtype, causal, n_split) in enumerate(CALLS):
        print(f"[noalloc] call {i}: B{B} H{H} Sq{Sq} Sk{Sk} D{D} {dtype} causal={causal} n_split={n_split}",
              flush=True)
        need = fa.split_workspace_size(B, H, Sq, Sk, D, n_split)
        assert 0 < need <= fa.SPLIT_SCRATCH_BYTES
        seed = 700 + i
        q, k, v = (fi.tensor_bits(seed, t, (B, H, S, D), dtype) for t, S in (("q", Sq), ("k", Sk), ("v", Sk)))
        tdt = torch.float16 if dtype == "f16" else torch.bfloat16
        qd, kd, vd = (torch.from_numpy(x.view(np.int16)).view(tdt).cuda() for x in (q, k, v))
        scale = 1.0 / math.sqrt(D)
        o_ref_split, l_ref_split = fa.fwd_split(qd, kd, vd, causal=causal, scale=scale, n_split=n_split)
        o = torch.full_like(qd, float("nan"))
        lse = torch.full((B, H, Sq), float("nan"), dtype=torch.float32, device="cuda")
        dt = fa.FA_F16 if dtype == "f16" else fa.FA_BF16
        st = fa.fa_fwd_split_noalloc(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                     B, H, Sq, Sk, D, scale, int(causal), dt, n_split, stream)
        assert st == fa.FA_OK, fa.fa_status_string(st)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_ref_split.view(torch.int16)), f"call {i}: O differs"
        assert torch.equal(lse.view(torch.int32), l_ref_split.view(torch.int32)), f"call {i}: lse differs"
        o_ref, l_ref = oracle_mod.attention(q, k, v, dtype, scale, causal, threads=THREADS)
        err_o = float(np.abs(o.double().cpu().numpy() - o_ref).max())
        err_l = float((np.abs(lse.double().cpu().numpy() - l_ref) / np.maximum(np.abs(l_ref), 1.0)).max())
        print(f"[noalloc] call {i}: bitwise equal to fa_fwd_split; max|dO| {err_o:.2e}, lse error {err_l:.2e}",
              flush=True)
        assert err_o <= TOL_O[dtype] and err_l <= TOL_LSE


def test_noalloc_too_large_launches_nothing():
    import torch

    from tile_level_programming_amd import fa

    B, H, Sq, Sk, D = 1, 1, 70000, 1024, 128
    q = torch.zeros(B, H, Sq, D, dtype=torch.float16, device="cuda")
    kv = torch.zeros(B, H, Sk, D, dtype=torch.float16, device="cuda")
    o = torch.full_like(q, 7.0)
    lse = torch.full((B, H, Sq), 7.0, dtype=torch.float32, device="cuda")
    st = fa.fa_fwd_split_noalloc(q.data_ptr(), kv.data_ptr(), kv.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                 B, H, Sq, Sk, D, 0.1, 0, fa.FA_F16, 4, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == fa.FA_ERR_SCRATCH_TOO_SMALL
    assert bool((o == 7).all()) and bool((lse == 7).all())

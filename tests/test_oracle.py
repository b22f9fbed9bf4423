"""Pins for the float64 oracle: exhaustive decoding, closed forms, invariants,
brute force on tiny inputs and a library cross-check.  Each test is chosen so
that a plausible slip in the oracle (a dropped scale, a flipped mask, a wrong
index or transposed operand, a missing max term in the lse) fails it."""

import math

import numpy as np
import pytest
import torch

import fa_inputs as fi


def _bits(x, dtype):
    """Exact float64 values -> uint16 patterns (values must be representable)."""
    x = np.asarray(x, dtype=np.float64)
    b = fi.f32_to_bits(x.astype(np.float32), dtype)
    return b


def _vals(bits, dtype):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    t = t.view(torch.float16 if dtype == "f16" else torch.bfloat16)
    return t.double().numpy()


def _rand(shape, dtype, seed, sigma=1.0):
    return fi.tensor_bits(seed, "q", shape, dtype, sigma)


# --- decoding ---------------------------------------------------------------


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_decode_exhaustive(oracle_mod, dtype):
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle_mod.decode(allbits, dtype)
    want = _vals(allbits, dtype)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    # sign of zero
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


# --- closed forms -----------------------------------------------------------


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_single_key(oracle_mod, dtype, causal):
    # Sk = 1: every row sees key 0 only, so O = v0 and lse = scale * q.k0
    B, H, Sq, D = 2, 3, 5, 16
    q = _rand((B, H, Sq, D), dtype, 1)
    k = fi.tensor_bits(1, "k", (B, H, 1, D), dtype)
    v = fi.tensor_bits(1, "v", (B, H, 1, D), dtype)
    scale = 0.37
    o, lse = oracle_mod.attention(q, k, v, dtype, scale, causal)
    qv, kv, vv = _vals(q, dtype), _vals(k, dtype), _vals(v, dtype)
    assert np.array_equal(o, np.broadcast_to(vv, o.shape))
    want = scale * np.einsum("bhid,bhd->bhi", qv, kv[:, :, 0, :])
    np.testing.assert_allclose(lse, want, rtol=1e-13, atol=1e-13)


def test_two_keys_closed_form(oracle_mod):
    # Sk = 2: O = sigmoid(s0 - s1) v0 + sigmoid(s1 - s0) v1, lse = logaddexp(s0, s1)
    dtype = "f16"
    B, H, Sq, D = 1, 2, 7, 8
    q = _rand((B, H, Sq, D), dtype, 2)
    k = fi.tensor_bits(2, "k", (B, H, 2, D), dtype)
    v = fi.tensor_bits(2, "v", (B, H, 2, D), dtype)
    scale = 1.7
    o, lse = oracle_mod.attention(q, k, v, dtype, scale, False)
    qv, kv, vv = _vals(q, dtype), _vals(k, dtype), _vals(v, dtype)
    for h in range(H):
        for i in range(Sq):
            s0 = scale * float(np.dot(qv[0, h, i], kv[0, h, 0]))
            s1 = scale * float(np.dot(qv[0, h, i], kv[0, h, 1]))
            w0 = 1.0 / (1.0 + math.exp(s1 - s0))
            w1 = 1.0 / (1.0 + math.exp(s0 - s1))
            np.testing.assert_allclose(o[0, h, i], w0 * vv[0, h, 0] + w1 * vv[0, h, 1], rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(lse[0, h, i], np.logaddexp(s0, s1), rtol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("how", ["zero_q", "zero_scale"])
def test_uniform_weights(oracle_mod, causal, how):
    # Q = 0 or scale = 0: every visible key has weight 1/n, lse = ln n
    dtype = "bf16"
    B, H, Sq, Sk, D = 1, 2, 9, 6, 8
    q = _rand((B, H, Sq, D), dtype, 3)
    if how == "zero_q":
        q[:] = 0
        scale = 0.5
    else:
        scale = 0.0
    k = fi.tensor_bits(3, "k", (B, H, Sk, D), dtype)
    v = fi.tensor_bits(3, "v", (B, H, Sk, D), dtype)
    o, lse = oracle_mod.attention(q, k, v, dtype, scale, causal)
    vv = _vals(v, dtype)
    for i in range(Sq):
        n = min(i + 1, Sk) if causal else Sk
        np.testing.assert_allclose(o[:, :, i], vv[:, :, :n].mean(axis=2), rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(lse[:, :, i], math.log(n), rtol=1e-14)


def test_large_logits_stable(oracle_mod):
    # logits near 1e4: exp without the max term would overflow; closed form holds
    dtype = "f16"
    q = _bits(np.full((1, 1, 1, 4), 50.0), dtype)
    k = _bits(np.array([[[[50.0, 50.0, 50.0, 50.0], [49.0, 50.0, 50.0, 50.0]]]]), dtype)
    v = _bits(np.array([[[[1.0, 0, 0, 0], [0, 1.0, 0, 0]]]]), dtype)
    o, lse = oracle_mod.attention(q, k, v, dtype, 1.0, False)
    s0, s1 = 10000.0, 9950.0
    assert np.all(np.isfinite(o)) and np.isfinite(lse).all()
    w1 = math.exp(s1 - s0) / (1 + math.exp(s1 - s0))
    np.testing.assert_allclose(o[0, 0, 0], [1 - w1, w1, 0, 0], rtol=1e-12, atol=1e-30)
    np.testing.assert_allclose(lse[0, 0, 0], np.logaddexp(s0, s1), rtol=1e-15)


# --- invariants -------------------------------------------------------------


@pytest.mark.parametrize("causal", [False, True])
def test_constant_v(oracle_mod, causal):
    dtype = "f16"
    B, H, S, D = 1, 2, 33, 16
    q = _rand((B, H, S, D), dtype, 4, 2.0)
    k = fi.tensor_bits(4, "k", (B, H, S, D), dtype, 2.0)
    row = fi.tensor_bits(4, "v", (B, H, 1, D), dtype)
    v = np.ascontiguousarray(np.broadcast_to(row, (B, H, S, D)))
    o, _ = oracle_mod.attention(q, k, v, dtype, 0.25, causal)
    np.testing.assert_allclose(o, np.broadcast_to(_vals(row, dtype), o.shape), rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_causal_is_prefix_attention(oracle_mod, dtype):
    # causal row i == non-causal attention over keys 0..i; rows i >= Sk see all keys
    B, H, Sq, Sk, D = 1, 1, 12, 9, 8
    q = _rand((B, H, Sq, D), dtype, 5)
    k = fi.tensor_bits(5, "k", (B, H, Sk, D), dtype)
    v = fi.tensor_bits(5, "v", (B, H, Sk, D), dtype)
    o, lse = oracle_mod.attention(q, k, v, dtype, 0.4, True)
    for i in range(Sq):
        n = min(i + 1, Sk)
        oi, li = oracle_mod.attention(q[:, :, i:i + 1], np.ascontiguousarray(k[:, :, :n]),
                                      np.ascontiguousarray(v[:, :, :n]), dtype, 0.4, False)
        np.testing.assert_allclose(o[:, :, i], oi[:, :, 0], rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(lse[:, :, i], li[:, :, 0], rtol=1e-14)


def test_causal_differs_from_noncausal(oracle_mod):
    # guards against a mask that never fires
    dtype = "f16"
    q = _rand((1, 1, 8, 8), dtype, 6)
    k = fi.tensor_bits(6, "k", (1, 1, 8, 8), dtype)
    v = fi.tensor_bits(6, "v", (1, 1, 8, 8), dtype)
    oc, _ = oracle_mod.attention(q, k, v, dtype, 0.5, True)
    on, _ = oracle_mod.attention(q, k, v, dtype, 0.5, False)
    np.testing.assert_allclose(oc[0, 0, 7], on[0, 0, 7], rtol=1e-14)  # last row sees everything
    np.testing.assert_array_equal(oc[0, 0, 0], _vals(v, dtype)[0, 0, 0])  # first row sees key 0
    assert np.abs(oc[0, 0, :7] - on[0, 0, :7]).max() > 1e-3


def test_key_permutation_invariance(oracle_mod):
    dtype = "bf16"
    B, H, S, D = 2, 2, 40, 16
    q = _rand((B, H, S, D), dtype, 7)
    k = fi.tensor_bits(7, "k", (B, H, S, D), dtype)
    v = fi.tensor_bits(7, "v", (B, H, S, D), dtype)
    perm = np.random.default_rng(1).permutation(S)
    o, lse = oracle_mod.attention(q, k, v, dtype, 0.3, False)
    o2, lse2 = oracle_mod.attention(q, np.ascontiguousarray(k[:, :, perm]), np.ascontiguousarray(v[:, :, perm]),
                                    dtype, 0.3, False)
    np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse2, lse, rtol=1e-13)


def test_key_translation(oracle_mod):
    # k_j -> k_j + u for every j: O unchanged, lse shifted by scale * q.u.
    # Small integers keep every input exact in fp16.
    dtype = "f16"
    rng = np.random.default_rng(2)
    B, H, S, D = 1, 2, 10, 8
    qv = rng.integers(-3, 4, size=(B, H, S, D)).astype(np.float64)
    kv = rng.integers(-3, 4, size=(B, H, S, D)).astype(np.float64)
    vv = rng.integers(-3, 4, size=(B, H, S, D)).astype(np.float64)
    u = rng.integers(-2, 3, size=(D,)).astype(np.float64)
    scale = 0.125
    o, lse = oracle_mod.attention(_bits(qv, dtype), _bits(kv, dtype), _bits(vv, dtype), dtype, scale, False)
    o2, lse2 = oracle_mod.attention(_bits(qv, dtype), _bits(kv + u, dtype), _bits(vv, dtype), dtype, scale, False)
    np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse2, lse + scale * (qv @ u), rtol=1e-13, atol=1e-13)


def test_linear_in_v(oracle_mod):
    dtype = "f16"
    rng = np.random.default_rng(3)
    B, H, S, D = 1, 1, 16, 8
    q = _rand((B, H, S, D), dtype, 8)
    k = fi.tensor_bits(8, "k", (B, H, S, D), dtype)
    v1 = rng.integers(-8, 9, size=(B, H, S, D)).astype(np.float64)
    v2 = rng.integers(-8, 9, size=(B, H, S, D)).astype(np.float64)
    for causal in (False, True):
        o1, _ = oracle_mod.attention(q, k, _bits(v1, dtype), dtype, 0.5, causal)
        o2, _ = oracle_mod.attention(q, k, _bits(v2, dtype), dtype, 0.5, causal)
        o3, _ = oracle_mod.attention(q, k, _bits(3 * v1 - 2 * v2, dtype), dtype, 0.5, causal)
        np.testing.assert_allclose(o3, 3 * o1 - 2 * o2, rtol=1e-12, atol=1e-12)


# --- brute force and a library cross-check ----------------------------------


def _brute_force(qv, kv, vv, scale, causal):
    """Independent naive attention in extended precision: no max subtraction,
    a different loop nest (keys outer), explicit boolean visibility."""
    ld = np.longdouble
    B, H, Sq, D = qv.shape
    Sk = kv.shape[2]
    o = np.zeros((B, H, Sq, D), dtype=ld)
    lse = np.zeros((B, H, Sq), dtype=ld)
    for b in range(B):
        for h in range(H):
            num = np.zeros((Sq, D), dtype=ld)
            den = np.zeros(Sq, dtype=ld)
            for j in range(Sk):
                kj = kv[b, h, j].astype(ld)
                vj = vv[b, h, j].astype(ld)
                for i in range(Sq):
                    if causal and j > i:
                        continue
                    w = np.exp(ld(scale) * np.sum(qv[b, h, i].astype(ld) * kj))
                    num[i] += w * vj
                    den[i] += w
            o[b, h] = num / den[:, None]
            lse[b, h] = np.log(den)
    return o, lse


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 1, 1, 1, 1), (2, 2, 5, 7, 3), (1, 2, 8, 3, 4), (2, 1, 3, 8, 8)])
def test_brute_force(oracle_mod, dtype, causal, shape):
    B, H, Sq, Sk, D = shape
    q = fi.tensor_bits(9, "q", (B, H, Sq, D), dtype)
    k = fi.tensor_bits(9, "k", (B, H, Sk, D), dtype)
    v = fi.tensor_bits(9, "v", (B, H, Sk, D), dtype)
    scale = 0.6
    o, lse = oracle_mod.attention(q, k, v, dtype, scale, causal)
    ob, lb = _brute_force(_vals(q, dtype), _vals(k, dtype), _vals(v, dtype), scale, causal)
    np.testing.assert_allclose(o, ob.astype(np.float64), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lb.astype(np.float64), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_sdpa_float64(oracle_mod, causal):
    # The pages validate the fused kernel against PyTorch's scaled-dot-product
    # attention; the oracle reproduces that library routine in float64 on CPU.
    w = fi.WORKLOADS["tiny_b1h2_s128_d64_f16"]
    q, k, v = fi.make_inputs(w)
    o, lse = oracle_mod.attention(q, k, v, w.dtype, w.scale, causal, threads=4)
    qt, kt, vt = (torch.from_numpy(_vals(x, w.dtype)) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=w.scale, is_causal=causal)
    np.testing.assert_allclose(o, ref.numpy(), rtol=1e-12, atol=1e-14)
    s = (qt @ kt.transpose(-1, -2)) * w.scale
    if causal:
        s = s.masked_fill(torch.ones(128, 128, dtype=torch.bool).triu(1), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, -1).numpy(), rtol=1e-13)


def test_rows_subset_and_threads(oracle_mod):
    # any subset of rows, in any order, over any number of threads, gives the same values
    w = fi.WORKLOADS["tiny_b1h2_s128_d64_f16"]
    q, k, v = fi.make_inputs(w)
    o, lse = oracle_mod.attention(q, k, v, w.dtype, w.scale, True)
    rows = np.array([255, 0, 128, 7, 127, 64], dtype=np.int64)
    os_, ls_ = oracle_mod.attention_rows(q, k, v, w.dtype, w.scale, True, rows, threads=3)
    np.testing.assert_array_equal(os_, o.reshape(-1, 64)[rows])
    np.testing.assert_array_equal(ls_, lse.reshape(-1)[rows])
    ot, lt = oracle_mod.attention(q, k, v, w.dtype, w.scale, True, threads=7)
    np.testing.assert_array_equal(ot, o)
    np.testing.assert_array_equal(lt, lse)


# --- split over the keys: key ranges and the log-sum-exp merge --------------


@pytest.mark.parametrize("causal", [False, True])
def test_key_range_is_attention_over_sliced_keys(oracle_mod, causal):
    # keys a <= j < b only: for non-causal rows, and for causal rows that see
    # the whole range (i >= b-1), the same as the oracle on the sliced k and
    # v; a causal row a <= i < b-1 sees keys a..i; rows i < a see nothing
    dtype = "f16"
    B, H, Sq, Sk, D = 1, 2, 48, 40, 16
    q = _rand((B, H, Sq, D), dtype, 31)
    k = fi.tensor_bits(31, "k", (B, H, Sk, D), dtype)
    v = fi.tensor_bits(31, "v", (B, H, Sk, D), dtype)
    a, b = 9, 27
    o, lse = oracle_mod.attention_rows(q, k, v, dtype, 0.4, causal, key_range=(a, b))
    o, lse = o.reshape(B, H, Sq, D), lse.reshape(B, H, Sq)
    ks, vs = np.ascontiguousarray(k[:, :, a:b]), np.ascontiguousarray(v[:, :, a:b])
    os_, ls_ = oracle_mod.attention(q, ks, vs, dtype, 0.4, False)
    for i in range(Sq):
        if not causal or i >= b - 1:
            np.testing.assert_allclose(o[:, :, i], os_[:, :, i], rtol=1e-13, atol=1e-15)
            np.testing.assert_allclose(lse[:, :, i], ls_[:, :, i], rtol=1e-14)
        elif i >= a:
            n = i - a + 1
            oi, li = oracle_mod.attention(np.ascontiguousarray(q[:, :, i:i + 1]), np.ascontiguousarray(ks[:, :, :n]),
                                          np.ascontiguousarray(vs[:, :, :n]), dtype, 0.4, False)
            np.testing.assert_allclose(o[:, :, i], oi[:, :, 0], rtol=1e-13, atol=1e-15)
            np.testing.assert_allclose(lse[:, :, i], li[:, :, 0], rtol=1e-14)
        else:
            assert np.all(lse[:, :, i] == -np.inf) and np.all(o[:, :, i] == 0.0)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("cuts", [(0, 100), (0, 37, 100), (0, 5, 64, 65, 100), (0, 1, 2, 3, 100)])
def test_merge_of_key_ranges_is_full_attention(oracle_mod, causal, cuts):
    # the log-sum-exp merge of partials over disjoint key ranges that cover
    # all keys gives the unsplit result (causal: rows below a range's start
    # contribute empty parts)
    dtype = "bf16"
    B, H, Sq, Sk, D = 2, 1, 100, 100, 8
    q = _rand((B, H, Sq, D), dtype, 32, 2.0)
    k = fi.tensor_bits(32, "k", (B, H, Sk, D), dtype, 2.0)
    v = fi.tensor_bits(32, "v", (B, H, Sk, D), dtype)
    parts = [oracle_mod.attention_rows(q, k, v, dtype, 0.35, causal, key_range=(a, b))
             for a, b in zip(cuts[:-1], cuts[1:])]
    o, lse = oracle_mod.merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    of, lf = oracle_mod.attention(q, k, v, dtype, 0.35, causal)
    np.testing.assert_allclose(o.reshape(of.shape), of, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse.reshape(lf.shape), lf, rtol=1e-13, atol=1e-13)


def test_merge_closed_forms(oracle_mod):
    D = 3
    o1 = np.array([[1.0, 2.0, 3.0], [4.0, 5.0, 6.0], [7.0, 8.0, 9.0], [1.0, 1.0, 1.0]])
    o2 = np.array([[3.0, 2.0, 1.0], [0.0, 0.0, 0.0], [-1.0, 0.0, 1.0], [2.0, 2.0, 2.0]])
    l1 = np.array([0.5, 2.0, -np.inf, -np.inf])
    l2 = np.array([0.5, -np.inf, 1.0, -np.inf])
    o2[1] = 0.0
    o1[2] = o1[2] * 0  # empty parts hold o = 0
    o1[3] = o2[3] = 0.0
    o, lse = oracle_mod.merge(np.stack([o1, o2]), np.stack([l1, l2]))
    # equal weights: the mean, lse + ln 2
    np.testing.assert_allclose(o[0], [2.0, 2.0, 2.0], rtol=1e-15)
    assert lse[0] == pytest.approx(0.5 + math.log(2.0), rel=1e-15)
    # one empty part: the other passes through
    np.testing.assert_allclose(o[1], o1[1], rtol=1e-15)
    np.testing.assert_allclose(o[2], o2[2], rtol=1e-15)
    assert lse[1] == 2.0 and lse[2] == 1.0
    # all parts empty
    assert lse[3] == -np.inf and np.all(o[3] == 0.0)
    # weights e^{lse_g - lse}: lse 0 and ln 3 give weights 1/4 and 3/4
    o, lse = oracle_mod.merge(np.array([[[4.0] * D], [[8.0] * D]]), np.array([[0.0], [math.log(3.0)]]))
    np.testing.assert_allclose(o[0], [7.0] * D, rtol=1e-15)
    assert lse[0] == pytest.approx(math.log(4.0), rel=1e-15)


def test_merge_part_order_irrelevant(oracle_mod):
    rng = np.random.default_rng(5)
    G, R, D = 5, 7, 4
    op = rng.normal(size=(G, R, D))
    lp = rng.normal(size=(G, R)) * 10
    lp[1, 3] = -np.inf
    o, lse = oracle_mod.merge(op, lp)
    perm = rng.permutation(G)
    o2, lse2 = oracle_mod.merge(op[perm], lp[perm])
    np.testing.assert_allclose(o2, o, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lse2, lse, rtol=1e-14)

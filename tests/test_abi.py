"""Host-side checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments before touching the device (these
calls return before any HIP call, so they run without a GPU)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = []
    for fn in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(\w+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while", "for", "return")))


@pytest.fixture(scope="module")
def fa():
    from tile_level_programming_amd import fa as mod

    return mod


def test_header_declares_entry_points():
    assert _declared_functions() == ["fa_fwd", "fa_fwd_split", "fa_fwd_split_count", "fa_fwd_split_noalloc",
                                     "fa_fwd_split_workspace_size", "fa_lse_merge", "fa_status_string",
                                     "gemm_bias_gelu", "rmsnorm_silu", "row_softmax"]


def test_library_exports_every_declared_symbol(fa):
    lib = fa.library()
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_status_strings_total(fa):
    for st in (0, 1, 2, 3, -1, 4, 1000):
        s = fa.fa_status_string(st)
        assert isinstance(s, str) and s
    assert fa.fa_status_string(99) == "unknown status"


A = 1 << 20  # a fake, 16-byte aligned, never dereferenced device address


def _call(fa, **kw):
    args = dict(q=A, k=2 * A, v=3 * A, o=4 * A, lse=5 * A, B=1, H=1, Sq=16, Sk=16, D=64,
                scale=0.125, causal=0, dtype=fa.FA_F16, stream=0)
    args.update(kw)
    return fa.fa_fwd(**args)


@pytest.mark.parametrize("kw", [
    dict(q=0), dict(k=0), dict(v=0), dict(o=0), dict(lse=0),
    dict(q=A + 8), dict(k=2 * A + 2), dict(v=3 * A + 4), dict(o=4 * A + 1), dict(lse=5 * A + 2),
    dict(B=0), dict(H=0), dict(Sq=0), dict(Sk=0), dict(B=-1), dict(D=0),
    dict(scale=float("inf")), dict(scale=float("nan")), dict(scale=float("-inf")),
    dict(Sq=1 << 25, D=64), dict(Sk=1 << 24, D=128), dict(B=1 << 16, H=1 << 16),
    dict(o=A), dict(o=3 * A + 512), dict(lse=2 * A), dict(lse=4 * A + 256),
])
def test_invalid_arguments(fa, kw):
    assert _call(fa, **kw) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(D=32), dict(D=96), dict(D=256), dict(dtype=2), dict(dtype=-1)])
def test_unsupported(fa, kw):
    assert _call(fa, **kw) == fa.FA_ERR_UNSUPPORTED


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    import importlib

    from tile_level_programming_amd import fa as mod

    monkeypatch.setattr(mod, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(ImportError):
        mod._load()


# --- split over the keys and the merge: host-side plan and checks ------------


@pytest.mark.parametrize("B,H,Sq,Sk,n_req,want", [
    (1, 1, 1, 64, 0, 1),          # too few keys to split
    (1, 1, 1, 1000, 1, 1),
    (1, 1, 1, 1000, 4, 4),        # chunk 256
    (1, 1, 1, 1000, 3, 3),        # chunk 384: 384, 384, 232
    (1, 1, 1, 100, 7, 2),         # at most one range per 64 keys: chunk 64
    (2, 32, 1, 16384, 0, 32),     # auto: 2048 / 64 work-groups
    (2, 32, 1, 4096, 0, 16),      # auto, capped at Sk / 256
    (2, 32, 8192, 8192, 0, 1),    # 4096 work-groups already
    (1, 4, 300, 65536, 0, 171),   # auto 2048/12 = 171 ranges of 384 keys
])
def test_split_count(fa, B, H, Sq, Sk, n_req, want):
    n = fa.split_count(B, H, Sq, Sk, n_req)
    assert n == want
    chunk = -(-Sk // n)
    assert n * chunk >= Sk
    for D in (64, 128):
        assert fa.split_workspace_size(B, H, Sq, Sk, D, n_req) == n * B * H * Sq * (D + 1) * 4


def test_split_count_invalid(fa):
    assert fa.split_count(0, 1, 1, 100, 0) == 0
    assert fa.split_count(1, 1, 1, 100, -1) == 0
    assert fa.split_workspace_size(1, 1, 1, 0, 64, 0) == 0


W = 64 * A  # fake workspace address


def _call_split(fa, **kw):
    args = dict(q=A, k=2 * A, v=3 * A, o=4 * A, lse=5 * A, B=1, H=1, Sq=16, Sk=1024, D=64,
                scale=0.125, causal=0, dtype=fa.FA_F16, n_split=4, workspace=W, workspace_bytes=1 << 20,
                stream=0)
    args.update(kw)
    return fa.fa_fwd_split(**args)


@pytest.mark.parametrize("kw", [
    dict(q=0), dict(lse=0), dict(o=A + 8), dict(Sk=0), dict(scale=float("nan")),
    dict(n_split=-1), dict(workspace=0), dict(workspace=W + 8),
    dict(workspace_bytes=4 * 16 * 65 * 4 - 1),           # one byte short
    dict(workspace=A - 4096),                            # overlaps q
    dict(workspace=4 * A), dict(workspace=5 * A - 1024),  # overlaps o, lse
])
def test_split_invalid_arguments(fa, kw):
    assert _call_split(fa, **kw) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(D=96), dict(dtype=2)])
def test_split_unsupported(fa, kw):
    assert _call_split(fa, **kw) == fa.FA_ERR_UNSUPPORTED


def _call_noalloc(fa, **kw):
    args = dict(q=A, k=2 * A, v=3 * A, o=4 * A, lse=5 * A, B=1, H=1, Sq=16, Sk=1024, D=64,
                scale=0.125, causal=0, dtype=fa.FA_F16, n_split=4, stream=0)
    args.update(kw)
    return fa.fa_fwd_split_noalloc(**args)


@pytest.mark.parametrize("kw", [
    dict(q=0), dict(lse=0), dict(o=A + 8), dict(Sk=0), dict(B=0), dict(scale=float("inf")),
    dict(n_split=-1), dict(o=A), dict(lse=3 * A + 64),  # outputs overlapping inputs
])
def test_noalloc_invalid_arguments(fa, kw):
    assert _call_noalloc(fa, **kw) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(D=96), dict(dtype=2)])
def test_noalloc_unsupported(fa, kw):
    assert _call_noalloc(fa, **kw) == fa.FA_ERR_UNSUPPORTED


def test_noalloc_rejects_partials_beyond_the_scratch(fa):
    # these checks return before any HIP call, so they run without a GPU
    B, H, Sq, Sk, D = 1, 1, 100000, 1024, 128
    assert fa.split_workspace_size(B, H, Sq, Sk, D, 4) > fa.SPLIT_SCRATCH_BYTES
    st = _call_noalloc(fa, o=64 * A, lse=128 * A, B=B, H=H, Sq=Sq, Sk=Sk, D=D, n_split=4)
    assert st == fa.FA_ERR_SCRATCH_TOO_SMALL
    assert "scratch" in fa.fa_status_string(st)


def _call_merge(fa, **kw):
    args = dict(o_parts=A, lse_parts=2 * A, n_part=3, rows=100, D=64, o=3 * A, lse=4 * A, dtype=fa.FA_BF16,
                stream=0)
    args.update(kw)
    return fa.fa_lse_merge(**args)


@pytest.mark.parametrize("kw", [
    dict(o_parts=0), dict(lse_parts=0), dict(o=0), dict(lse=0),
    dict(o_parts=A + 4), dict(o=3 * A + 8), dict(lse=4 * A + 2),
    dict(n_part=0), dict(rows=0), dict(D=0),
    dict(o=A + 3 * 100 * 64 * 4 - 16),                 # overlaps the O parts
    dict(lse=2 * A + 8),                               # overlaps the lse parts
    dict(lse=3 * A + 100 * 64 * 2 - 4),                # overlaps o
])
def test_merge_invalid_arguments(fa, kw):
    assert _call_merge(fa, **kw) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(D=32), dict(D=256), dict(dtype=5)])
def test_merge_unsupported(fa, kw):
    assert _call_merge(fa, **kw) == fa.FA_ERR_UNSUPPORTED


# --- GEMM with the fused bias + GELU epilogue: host-side checks --------------


def _call_gemm(fa, **kw):
    args = dict(a=A, w=2 * A, bias=3 * A, c=4 * A, M=100, N=64, K=64, dtype=fa.FA_F16, stream=0)
    args.update(kw)
    return fa.gemm_bias_gelu(**args)


@pytest.mark.parametrize("kw", [
    dict(a=0), dict(w=0), dict(c=0), dict(a=A + 8), dict(w=2 * A + 4), dict(c=4 * A + 2), dict(bias=3 * A + 1),
    dict(M=0), dict(N=0), dict(K=0), dict(M=-5), dict(M=1 << 31), dict(K=1 << 24),
    dict(c=A + 96), dict(c=2 * A - 64), dict(c=3 * A - 16),   # overlaps a, w, bias
])
def test_gemm_invalid_arguments(fa, kw):
    assert _call_gemm(fa, **kw) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(K=12), dict(K=100), dict(dtype=3)])
def test_gemm_unsupported(fa, kw):
    assert _call_gemm(fa, **kw) == fa.FA_ERR_UNSUPPORTED


# --- row-wise kernels: host-side checks ----------------------------------------


@pytest.mark.parametrize("kw", [dict(x=0), dict(y=0), dict(x=A + 1), dict(y=2 * A + 3), dict(R=0), dict(C=0),
                                dict(R=1 << 31), dict(y=A + 64)])
def test_row_softmax_invalid(fa, kw):
    args = dict(x=A, y=2 * A, R=100, C=500, dtype=fa.FA_F16, stream=0)
    args.update(kw)
    assert fa.row_softmax(**args) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(C=32769), dict(dtype=2)])
def test_row_softmax_unsupported(fa, kw):
    args = dict(x=A, y=2 * A, R=100, C=500, dtype=fa.FA_F16, stream=0)
    args.update(kw)
    assert fa.row_softmax(**args) == fa.FA_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw", [dict(g=0), dict(g=3 * A + 1), dict(eps=-1.0), dict(eps=float("nan")),
                                dict(eps=float("inf")), dict(g=2 * A + 64), dict(x=0)])
def test_rmsnorm_silu_invalid(fa, kw):
    args = dict(x=A, g=3 * A, y=2 * A, R=100, C=500, eps=1e-6, dtype=fa.FA_BF16, stream=0)
    args.update(kw)
    assert fa.rmsnorm_silu(**args) == fa.FA_ERR_INVALID_ARG



# --- the torch-level helpers check caller-supplied outputs before any call ---


def test_output_checks_on_host_tensors(fa):
    import torch

    dev = torch.device("cuda", 0)
    good = dict(shape=(2, 3), dtype=torch.float16, device=dev)
    with pytest.raises(TypeError):
        fa._check_out(object(), "out", **good)
    with pytest.raises(TypeError):
        fa._check_out(torch.empty(2, 3, dtype=torch.float32), "out", **good)
    with pytest.raises(ValueError):
        fa._check_out(torch.empty(2, 4, dtype=torch.float16), "out", **good)
    with pytest.raises(ValueError):  # right shape and type, but host memory
        fa._check_out(torch.empty(2, 3, dtype=torch.float16), "out", **good)


def test_helpers_reject_host_inputs(fa):
    import torch

    q = torch.zeros(1, 1, 8, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        fa.fwd(q, q, q)
    with pytest.raises(ValueError):
        fa.fwd_split(q, q, q)
    with pytest.raises(ValueError):
        fa.linear_gelu(torch.zeros(4, 8, dtype=torch.float16), torch.zeros(4, 8, dtype=torch.float16))
    with pytest.raises(ValueError):
        fa.softmax(torch.zeros(4, 8, dtype=torch.float16))
    with pytest.raises(ValueError):
        fa.lse_merge(torch.zeros(2, 3, 64), torch.zeros(2, 3), torch.float16)

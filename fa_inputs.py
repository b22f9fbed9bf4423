"""Seeded synthetic inputs for the fused attention forward pass.

This module is shared by the float64 oracle's tests, the GPU parity tests and
the benchmark.  It holds no attention arithmetic: it only draws i.i.d. normal
values from a counter-based generator and rounds them to fp16/bf16 bit
patterns, and it names the workloads (shapes, dtype, mask mode, seed, sigma).

Generator (its own definition, stated here so that any reader can re-derive
every input bit):

* SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014): the n-th output (n = 0, 1, ...) of the sequence
  seeded with ``s`` is ``mix(s + (n + 1) * GAMMA)`` modulo 2**64, where
  ``mix`` is the variant-13 finaliser below.  Because the n-th output has this
  closed form, element ``i`` of a tensor can be drawn without drawing the ones
  before it.
* Stream key of a tensor: output 0 of SplitMix64 seeded with
  ``8 * seed + tensor_id`` (tensor_id: Q=0, K=1, V=2).
* Uniforms: ``u = ((z >> 11) + 1) * 2**-53`` lies in (0, 1].
* Element ``i`` (flat index in the contiguous [B, H, S, D] tensor) is the
  Box-Muller cosine branch of outputs ``2i`` and ``2i+1`` of its stream:
  ``sigma * sqrt(-2 ln u1) * cos(2 pi u2)``, computed in float64, rounded to
  float32 (round to nearest even) and then to the storage type (round to
  nearest even).

The pages that describe the method measure on no dataset; their attention
kernel is checked on random tensors.  The workloads below are the five
synthetic shapes the port is measured and checked on.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

GAMMA = 0x9E3779B97F4A7C15
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_MASK64 = (1 << 64) - 1

TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "a": 3, "w": 4, "bias": 5, "x": 6, "g": 7}  # attention; GEMM; row-wise
DTYPES = ("f16", "bf16")


def _mix(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def splitmix64_at(seed: int, n: np.ndarray) -> np.ndarray:
    """Outputs number ``n`` (uint64 array, 0-based) of SplitMix64 seeded with ``seed``."""
    n = np.asarray(n, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed & _MASK64) + (n + np.uint64(1)) * np.uint64(GAMMA)
        return _mix(z)


def stream_key(seed: int, tensor_id: int) -> int:
    return int(splitmix64_at(8 * seed + tensor_id, np.zeros(1, np.uint64))[0])


def normals(key: int, start: int, count: int) -> np.ndarray:
    """float64 N(0, 1) values for flat element indices start .. start+count-1."""
    idx = np.arange(start, start + count, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z1 = splitmix64_at(key, idx * np.uint64(2))
        z2 = splitmix64_at(key, idx * np.uint64(2) + np.uint64(1))
    two53 = 2.0 ** -53
    u1 = ((z1 >> np.uint64(11)).astype(np.float64) + 1.0) * two53
    u2 = ((z2 >> np.uint64(11)).astype(np.float64) + 1.0) * two53
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * math.pi * u2)


def f32_to_bits(x32: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to fp16 or bf16 (nearest even); return uint16 bit patterns."""
    x32 = np.asarray(x32, dtype=np.float32)
    if dtype == "f16":
        return x32.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        b = x32.view(np.uint32).astype(np.uint64)
        nan = np.isnan(x32)
        r = (b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
        r = r.astype(np.uint16)
        r[nan] = 0x7FC0
        return r
    raise ValueError(f"unknown dtype {dtype!r}")


def tensor_bits(seed: int, name: str, shape, dtype: str, sigma: float = 1.0,
                chunk: int = 1 << 22) -> np.ndarray:
    """uint16 bit patterns of one seeded input tensor, contiguous, shape ``shape``."""
    key = stream_key(seed, TENSOR_IDS[name])
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, chunk):
        c = min(chunk, n - s)
        x = normals(key, s, c) * sigma
        out[s:s + c] = f32_to_bits(x.astype(np.float32), dtype)
    return out.reshape(shape)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Sq: int
    Sk: int
    D: int
    dtype: str
    causal: bool
    seed: int
    sigma_qk: float = 1.0
    sigma_v: float = 1.0
    split: bool = False  # run through the key-split entry point (decode-shaped calls)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def shape_q(self):
        return (self.B, self.H, self.Sq, self.D)

    def shape_kv(self):
        return (self.B, self.H, self.Sk, self.D)

    def unmasked_pairs(self) -> int:
        """Number of (query, key) pairs the causal mask leaves visible, per (b, h)."""
        if not self.causal:
            return self.Sq * self.Sk
        # top-left alignment: query i sees keys 0..min(i, Sk-1)
        full = max(0, self.Sq - self.Sk)  # rows i >= Sk see all Sk keys
        m = min(self.Sq, self.Sk)
        return m * (m + 1) // 2 + full * self.Sk

    def flops(self) -> int:
        """Algorithmic FLOP of the two products (scores and P.V): 4*D per visible pair."""
        return 4 * self.B * self.H * self.D * self.unmasked_pairs()

    def io_bytes(self) -> int:
        """Q, K, V read once, O written once, lse written once."""
        e = 2
        return (e * self.B * self.H * (2 * self.Sq * self.D + 2 * self.Sk * self.D)
                + 4 * self.B * self.H * self.Sq)


# The five measured shapes.  Q, K, V are i.i.d. normal; the last one draws Q and
# K with variance 4 (sigma 2) to give large logits that stress the running-max
# rescale.  scale = 1/sqrt(D) throughout.
WORKLOADS = {
    "tiny_b1h2_s128_d64_f16": Workload("tiny_b1h2_s128_d64_f16", 1, 2, 128, 128, 64, "f16", False, 1),
    "causal_b2h8_s1024_d64_f16": Workload("causal_b2h8_s1024_d64_f16", 2, 8, 1024, 1024, 64, "f16", True, 2),
    "b4h16_s4096_d128_bf16": Workload("b4h16_s4096_d128_bf16", 4, 16, 4096, 4096, 128, "bf16", False, 3),
    "causal_b4h16_s4096_d128_bf16": Workload("causal_b4h16_s4096_d128_bf16", 4, 16, 4096, 4096, 128, "bf16", True, 3),
    "b2h32_s8192_d64_f16": Workload("b2h32_s8192_d64_f16", 2, 32, 8192, 8192, 64, "f16", False, 4),
    "causal_b1h32_s16384_d128_bf16_sigma2": Workload("causal_b1h32_s16384_d128_bf16_sigma2", 1, 32, 16384, 16384, 128,
                                                     "bf16", True, 5, sigma_qk=2.0, sigma_v=1.0),
}
HEADLINE = "b2h32_s8192_d64_f16"

# Decode-shaped calls (a few queries per head against a long key sequence),
# run through the key-split entry point: one work-group per (batch, head,
# query block) would occupy a small part of the GPU, and the time is the one
# pass over K and V, so these are HBM-bound.  Non-causal, i.i.d. normal.
DECODE_WORKLOADS = {
    "decode_b16h32_sq1_sk16384_d128_bf16": Workload("decode_b16h32_sq1_sk16384_d128_bf16", 16, 32, 1, 16384, 128,
                                                    "bf16", False, 6, split=True),
    "decode_b8h32_sq16_sk32768_d64_f16": Workload("decode_b8h32_sq16_sk32768_d64_f16", 8, 32, 16, 32768, 64,
                                                  "f16", False, 7, split=True),
}
ALL_WORKLOADS = {**WORKLOADS, **DECODE_WORKLOADS}


@dataclasses.dataclass(frozen=True)
class GemmWorkload:
    """C = gelu(A W^T + bias): A [M, K], W [N, K], bias [N], i.i.d. N(0, sigma^2)."""
    name: str
    M: int
    N: int
    K: int
    dtype: str
    seed: int
    sigma: float = 1.0
    bias: bool = True

    def flops(self) -> int:
        """Algorithmic FLOP of the product (the epilogue is not counted): 2*M*N*K."""
        return 2 * self.M * self.N * self.K

    def io_bytes(self) -> int:
        """A, W and bias read once, C written once."""
        return 2 * (self.M * self.K + self.N * self.K + (self.N if self.bias else 0) + self.M * self.N)


def make_gemm_inputs(w: GemmWorkload):
    """(a, w, bias or None) uint16 bit-pattern arrays for a GEMM workload.  The
    inputs are scaled by 1/sqrt(K) on the weight side, so that the
    pre-activations are O(1) as in a trained layer and the GELU is not
    saturated."""
    a = tensor_bits(w.seed, "a", (w.M, w.K), w.dtype, w.sigma)
    wt = tensor_bits(w.seed, "w", (w.N, w.K), w.dtype, w.sigma / math.sqrt(w.K))
    b = tensor_bits(w.seed, "bias", (w.N,), w.dtype, w.sigma) if w.bias else None
    return a, wt, b


@dataclasses.dataclass(frozen=True)
class RowWorkload:
    """A row-wise kernel on R rows of length C: op "softmax" (x ~ N(0, sigma^2))
    or "rmsnorm_silu" (x ~ N(0, sigma^2), weight g ~ N(0, 1), eps 1e-6)."""
    name: str
    op: str
    R: int
    C: int
    dtype: str
    seed: int
    sigma: float = 1.0
    eps: float = 1e-6

    def io_bytes(self) -> int:
        """x read once, y written once (and g read once)."""
        return 2 * 2 * self.R * self.C + (2 * self.C if self.op == "rmsnorm_silu" else 0)


def make_row_inputs(w: RowWorkload):
    """(x, g or None) uint16 bit-pattern arrays for a row-wise workload."""
    x = tensor_bits(w.seed, "x", (w.R, w.C), w.dtype, w.sigma)
    g = tensor_bits(w.seed, "g", (w.C,), w.dtype) if w.op == "rmsnorm_silu" else None
    return x, g


# Row-wise kernels.  The pages give no shapes; these are attention-score rows
# (4096 keys) and vocabulary-size rows (32000) for the softmax, and a VAE
# feature map (65536 positions x 512 channels) and transformer hidden states
# (16384 x 4096) for RMSNorm + SiLU.
ROW_WORKLOADS = {
    "softmax_r32768_c4096_f16": RowWorkload("softmax_r32768_c4096_f16", "softmax", 32768, 4096, "f16", 10, 3.0),
    "softmax_r8192_c32000_bf16": RowWorkload("softmax_r8192_c32000_bf16", "softmax", 8192, 32000, "bf16", 11, 3.0),
    "rmsnorm_silu_r65536_c512_bf16": RowWorkload("rmsnorm_silu_r65536_c512_bf16", "rmsnorm_silu", 65536, 512,
                                                 "bf16", 12),
    "rmsnorm_silu_r16384_c4096_f16": RowWorkload("rmsnorm_silu_r16384_c4096_f16", "rmsnorm_silu", 16384, 4096,
                                                 "f16", 13),
}


# GEMM with the fused bias + GELU epilogue.  The pages name no shapes (their
# example tile is 128 x 128 x 32); these are the up-projection of a
# transformer MLP (8192 tokens, 4096 -> 16384) and a square one.
GEMM_WORKLOADS = {
    "gemm_m8192_n16384_k4096_bf16": GemmWorkload("gemm_m8192_n16384_k4096_bf16", 8192, 16384, 4096, "bf16", 8),
    "gemm_m4096_n4096_k4096_f16": GemmWorkload("gemm_m4096_n4096_k4096_f16", 4096, 4096, 4096, "f16", 9),
}


def make_inputs(w: Workload):
    """(q, k, v) uint16 bit-pattern arrays for a workload."""
    q = tensor_bits(w.seed, "q", w.shape_q(), w.dtype, w.sigma_qk)
    k = tensor_bits(w.seed, "k", w.shape_kv(), w.dtype, w.sigma_qk)
    v = tensor_bits(w.seed, "v", w.shape_kv(), w.dtype, w.sigma_v)
    return q, k, v

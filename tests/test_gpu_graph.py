"""fa_fwd launched from a captured HIP graph: every replay equals an eager call, bit for bit.

The benchmark times launches shorter than the host's call rate from captured
graphs (kernel launches only, no memory-set nodes).  Here each replay is
checked on its own, with eager work and synchronisations between replays.
"""

import numpy as np
import pytest

import fa_inputs as fi

pytestmark = pytest.mark.gpu

SHAPES = [
    # (B, H, Sq, Sk, D, dtype, causal): two key groups (the small causal
    # workload and the tiny one), and a D=128 launch with a ragged end
    (2, 8, 1024, 1024, 64, "f16", True),
    (1, 2, 128, 128, 64, "f16", False),
    (1, 3, 1000, 1000, 128, "bf16", True),
]


@pytest.mark.parametrize("shape", SHAPES)
def test_graph_replays_equal_eager(shape):
    import torch

    from tile_level_programming_amd import fa

    B, H, Sq, Sk, D, dtype, causal = shape
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    seed = 900 + Sq + D

    def dev(name, shp):
        bits = fi.tensor_bits(seed, name, shp, dtype)
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(tdt).to("cuda")

    q, k, v = dev("q", (B, H, Sq, D)), dev("k", (B, H, Sk, D)), dev("v", (B, H, Sk, D))
    print(f"[graph] {shape}", flush=True)
    o_e, l_e = fa.fwd(q, k, v, causal=causal)
    torch.cuda.synchronize()

    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, Sq), float("nan"), dtype=torch.float32, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(3):
            fa.fwd(q, k, v, causal=causal, out=o, lse=lse)
    q2 = torch.flip(q, dims=[2]).contiguous()
    for rep in range(3):
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        fa.fwd(q2, k, v, causal=causal)  # eager work on other buffers between the replays
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_e.view(torch.int16)), f"replay {rep}: O differs from the eager call"
        assert torch.equal(lse.view(torch.int32), l_e.view(torch.int32)), f"replay {rep}: lse differs"


ROW_SHAPES = [
    # (op, R, C, dtype): one row per wave group, and rows spread over the work-group
    ("rmsnorm_silu", 4096, 512, "bf16"),
    ("softmax", 512, 4096, "f16"),
    ("softmax", 64, 32000, "bf16"),
]


@pytest.mark.parametrize("shape", ROW_SHAPES)
def test_graph_replays_equal_eager_rows(shape):
    import torch

    from tile_level_programming_amd import fa

    op, R, C, dtype = shape
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    gen = torch.Generator(device="cpu").manual_seed(R + C)
    x = torch.randn(R, C, generator=gen).to(tdt).to("cuda")
    g = torch.randn(C, generator=gen).to(tdt).to("cuda")
    x2 = torch.flip(x, dims=[0]).contiguous()

    def call(inp, out=None):
        return fa.softmax(inp, out=out) if op == "softmax" else fa.rmsnorm_silu_rows(inp, g, 1e-6, out=out)

    print(f"[graph] {shape}", flush=True)
    y_e = call(x)
    torch.cuda.synchronize()
    y = torch.full_like(x, float("nan"))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(3):
            call(x, out=y)
    for rep in range(3):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        call(x2)  # eager work on other buffers between the replays
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_e.view(torch.int16)), f"replay {rep}: output differs from the eager call"

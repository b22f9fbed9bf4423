"""The oracle against hand-derived closed-form cases stored in tests/golden/."""

import json
import os

import numpy as np
import pytest

import fa_inputs as fi

HERE = os.path.dirname(os.path.abspath(__file__))
DOC = json.load(open(os.path.join(HERE, "golden", "hand_cases.json")))


@pytest.mark.parametrize("case", DOC["cases"], ids=[c["name"] for c in DOC["cases"]])
def test_hand_case(oracle_mod, case):
    B, H, Sq, Sk, D = case["B"], case["H"], case["Sq"], case["Sk"], case["D"]
    dt = case["dtype"]

    def bits(vals, shape):
        return fi.f32_to_bits(np.asarray(vals, dtype=np.float32), dt).reshape(shape)

    q = bits(case["q"], (B, H, Sq, D))
    k = bits(case["k"], (B, H, Sk, D))
    v = bits(case["v"], (B, H, Sk, D))
    o, lse = oracle_mod.attention(q, k, v, dt, case["scale"], case["causal"])
    np.testing.assert_allclose(o.reshape(-1), [float(x) for x in case["o"]], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(lse.reshape(-1), [float(x) for x in case["lse"]], rtol=1e-14, atol=1e-15)

"""The oracle reproduces its stored regression fixtures (tests/golden)."""
import json
import os

import numpy as np
import pytest

import oracle as O
from synth import clustered_head, gaussian

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
with open(os.path.join(HERE, "oracle_regression.json")) as f:
    GOLD = json.load(f)


@pytest.mark.parametrize("name", sorted(GOLD))
def test_oracle_regression(name):
    g = GOLD[name]
    if g["kind"] == "gaussian":
        Q, K, V = gaussian(**g["shape"])
        q, k, v = Q[0], K[0], V[0]
    else:
        q, k, v = clustered_head(**g["shape"])
    q, k, v = (O.bf16_to_f64(x) for x in (q, k, v))
    o, l, info = O.sol_attn_head_ref(q, k, v, g["B"], g["beta"])
    np.testing.assert_array_equal(info["mask"].astype(int), np.array(g["mask"]))
    np.testing.assert_allclose(o, np.array(g["out"]), rtol=0, atol=1e-13)
    np.testing.assert_allclose(l, np.array(g["lse"]), rtol=0, atol=1e-13)

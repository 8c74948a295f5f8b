"""The oracles reproduce their stored regression fixtures (tests/golden): the
sparse head, key-share partials, 3D neighbourhood attention and the FP8
quantisation and GEMM."""
import json
import os

import numpy as np
import pytest

import oracle as O
import oracle.fp8 as F
import oracle.na3d as NA
from synth import activations, clustered_head, gaussian

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
with open(os.path.join(HERE, "oracle_regression.json")) as f:
    GOLD = json.load(f)


@pytest.mark.parametrize("name", sorted(GOLD))
def test_oracle_regression(name):
    g = GOLD[name]
    if g["kind"] == "share":
        Q, K, V = gaussian(heads=1, n=40, d=8, seed=g["seed"])
        q, k, v = (O.bf16_to_f64(x[0]) for x in (Q, K, V))
        _, _, info = O.sol_attn_head_ref(q, k, v, g["B"], g["beta"], blocks=g["blocks"])
        num, den, m = info["partial"]
        np.testing.assert_allclose(num, np.array(g["num"]), rtol=0, atol=1e-13)
        np.testing.assert_allclose(den, np.array(g["den"]), rtol=0, atol=1e-13)
        np.testing.assert_allclose(m, np.array(g["ref"]), rtol=0, atol=1e-13)
        return
    if g["kind"] == "na3d":
        Q, K, V = gaussian(heads=1, n=int(np.prod(g["grid"])), d=8, seed=g["seed"])
        o, l = NA.na3d_head_ref(*(O.bf16_to_f64(x[0]) for x in (Q, K, V)), g["grid"], g["window"])
        np.testing.assert_allclose(o, np.array(g["out"]), rtol=0, atol=1e-13)
        np.testing.assert_allclose(l, np.array(g["lse"]), rtol=0, atol=1e-13)
        return
    if g["kind"] == "fp8":
        qa, sa = F.quantize_rows_ref(activations(6, 32, seed=g["seeds"][0]))
        qw, sw = F.quantize_rows_ref(activations(5, 32, seed=g["seeds"][1]))
        np.testing.assert_array_equal(qa.astype(int), np.array(g["codes_a"]))
        np.testing.assert_array_equal(qw.astype(int), np.array(g["codes_w"]))
        np.testing.assert_array_equal(sa.astype(float), np.array(g["scale_a"]))
        np.testing.assert_array_equal(sw.astype(float), np.array(g["scale_w"]))
        y, _ = F.fp8_gemm_ref(qa, sa, qw, sw)
        np.testing.assert_array_equal(y, np.array(g["y"]))  # exact: integer dot products, scaled
        return
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

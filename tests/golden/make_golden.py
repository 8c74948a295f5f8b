"""Writes the oracle regression fixtures in this folder.

Calls only ``oracle`` (and the seeded input generator ``synth``).  The pages
print no worked numeric example for the method, so these fixtures pin the
oracle against its own earlier, reviewed output: any later change of its
arithmetic shows up as a diff here and has to name the passage that justifies it.

Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle as O  # noqa: E402
import oracle.fp8 as F  # noqa: E402
import oracle.na3d as NA  # noqa: E402
from synth import activations, clustered_head, gaussian  # noqa: E402

CASES = [
    # name, generator, shape, B, beta
    ("gauss_h1_n40_d8_b8_beta0.5", "gaussian", dict(heads=1, n=40, d=8, seed=21), 8, 0.5),
    ("gauss_h1_n37_d8_b8_beta0", "gaussian", dict(heads=1, n=37, d=8, seed=22), 8, 0.0),
    ("clustered_n48_d16_b8_beta1", "clustered", dict(n=48, d=16, block=8, centres=4,
                                                    noise=0.5, seed=23, h=0), 8, 1.0),
]


def inputs(kind, shape):
    if kind == "gaussian":
        Q, K, V = gaussian(**shape)
        return Q[0], K[0], V[0]
    return clustered_head(**shape)


def main():
    out = {}
    for name, kind, shape, B, beta in CASES:
        q, k, v = (O.bf16_to_f64(x) for x in inputs(kind, shape))
        o, l, info = O.sol_attn_head_ref(q, k, v, B, beta)
        out[name] = dict(kind=kind, shape=shape, B=B, beta=beta,
                         out=np.round(o, 15).tolist(), lse=np.round(l, 15).tolist(),
                         mask=info["mask"].astype(int).tolist())
    # key-share partials (unnormalised numerator, denominator, reference) of
    # two block ranges of one sequence
    for name, blocks in (("share_gauss_n40_d8_b8_blocks0-2", [0, 1, 2]),
                         ("share_gauss_n40_d8_b8_blocks3-4", [3, 4])):
        q, k, v = (O.bf16_to_f64(x) for x in inputs("gaussian", dict(heads=1, n=40, d=8, seed=24)))
        _, _, info = O.sol_attn_head_ref(q, k, v, 8, 0.5, blocks=blocks)
        num, den, m = info["partial"]
        out[name] = dict(kind="share", seed=24, blocks=blocks, B=8, beta=0.5,
                         num=np.round(num, 15).tolist(), den=np.round(den, 15).tolist(),
                         ref=np.round(m, 15).tolist())
    # 3D neighbourhood attention on a small grid with windows clamped at every border
    grid, window = (3, 4, 5), (3, 3, 3)
    Q, K, V = gaussian(heads=1, n=int(np.prod(grid)), d=8, seed=25)
    o, l = NA.na3d_head_ref(*(O.bf16_to_f64(x[0]) for x in (Q, K, V)), grid, window)
    out["na3d_grid3x4x5_win3x3x3_d8"] = dict(kind="na3d", seed=25, grid=grid, window=window,
                                             out=np.round(o, 15).tolist(), lse=np.round(l, 15).tolist())
    # FP8: row quantisation of bf16 activations and the row-scaled GEMM
    x = activations(6, 32, seed=26)
    w = activations(5, 32, seed=27)
    qa, sa = F.quantize_rows_ref(x)
    qw, sw = F.quantize_rows_ref(w)
    y, _ = F.fp8_gemm_ref(qa, sa, qw, sw)
    out["fp8_m6_n5_k32"] = dict(kind="fp8", seeds=[26, 27], codes_a=qa.astype(int).tolist(),
                                scale_a=sa.astype(float).tolist(), codes_w=qw.astype(int).tolist(),
                                scale_w=sw.astype(float).tolist(), y=y.tolist())
    with open(os.path.join(HERE, "oracle_regression.json"), "w") as f:
        json.dump(out, f, indent=0)


if __name__ == "__main__":
    main()

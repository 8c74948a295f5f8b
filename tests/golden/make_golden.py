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
from synth import gaussian, clustered_head  # noqa: E402

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
    with open(os.path.join(HERE, "oracle_regression.json"), "w") as f:
        json.dump(out, f, indent=0)


if __name__ == "__main__":
    main()

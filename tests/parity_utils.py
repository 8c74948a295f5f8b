"""Shared helpers of the GPU parity tests: device transfer, tolerances, and the
oracle comparison that accepts either decision on near-tie pairs.

The oracle never receives anything computed by the HIP path: the set of
near-tie pairs comes from the oracle's own proxy scores and thresholds, and
for each such pair both decisions are evaluated by the oracle.
"""
import itertools
import math
from collections import defaultdict

import numpy as np

import oracle as O

# Output tolerances for unit-scale V: max abs <= 1e-2, mean abs <= 1e-3.
OUT_MAX = 1e-2
OUT_MEAN = 1e-3
LSE_MAX = 1e-3
# Pairs whose oracle proxy lies within this distance of the threshold may be
# decided either way.
TIE_EPS = 1e-4


def dev(bits):
    """uint16 bf16 bits (numpy) -> torch bf16 tensor on the GPU."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def host(t):
    """GPU tensor -> float64 numpy (bf16 values are exact)."""
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def tiles_rows(n, which=("first", "mid", "last"), tile=128):
    """Query rows of a few whole 128-row tiles (first, middle, last)."""
    nqt = (n + tile - 1) // tile
    pick = {"first": 0, "mid": nqt // 2, "last": nqt - 1}
    rows = []
    for w in which:
        t = pick[w]
        rows.extend(range(t * tile, min(n, (t + 1) * tile)))
    return np.array(sorted(set(rows)), dtype=np.int64)


def sparse_with_ties(q, k, v, B, beta, rows, eps=TIE_EPS, max_ties=6, gpu_mask=None):
    """Oracle output for ``rows`` plus, for rows with near-ties, the outputs under
    every combination of decisions on their near-tie pairs.

    A row with more than ``max_ties`` near-tie pairs is not enumerated: its
    reference takes the GPU's own decisions on those pairs (``gpu_mask``, bool
    ``[len(rows), nb]``, the selection the GPU computed for the same rows), the
    reading the tie tolerance allows; the caller checks separately that the GPU
    mask agrees with the oracle's everywhere outside the tie band.  Without a
    GPU mask such a row is an error rather than a silently partial reference."""
    out, lse, info = O.sol_attn_head_ref(q, k, v, B, beta, rows=rows)
    ties = O.near_ties_ref(info["p"], info["mu"], info["sigma"], beta, eps)
    by_row = defaultdict(list)
    for i, j in ties:
        by_row[i].append(j)
    cands = {}
    for i, js in by_row.items():
        if len(js) > max_ties:
            assert gpu_mask is not None, (
                f"row {int(rows[i])}: {len(js)} near-tie pairs exceed the enumeration cap "
                f"{max_ties}; pass the GPU mask")
            force = {(int(rows[i]), j): bool(gpu_mask[i][j]) for j in js}
            o, l, _ = O.sol_attn_head_ref(q, k, v, B, beta, rows=[int(rows[i])], force=force,
                                          pooled=info["pooled"])
            cands[i] = [(o[0], l[0])]
            continue
        opts = []
        base = info["mask"][i]
        for bits in itertools.product([False, True], repeat=len(js)):
            if all(b == bool(base[j]) for b, j in zip(bits, js)):
                opts.append((out[i], lse[i]))
                continue
            force = {(int(rows[i]), j): b for j, b in zip(js, bits)}
            o, l, _ = O.sol_attn_head_ref(q, k, v, B, beta, rows=[int(rows[i])], force=force,
                                          pooled=info["pooled"])
            opts.append((o[0], l[0]))
        cands[i] = opts
    return out, lse, info, cands


def best_match(gpu_out, gpu_lse, out, lse, cands):
    """Per-row oracle reference, picking for near-tie rows the candidate closest to
    the GPU row (any of them is a correct answer)."""
    ref_o = out.copy()
    ref_l = lse.copy()
    for i, opts in cands.items():
        errs = [np.abs(gpu_out[i] - o).max() for o, _ in opts]
        b = int(np.argmin(errs))
        ref_o[i] = opts[b][0]
        ref_l[i] = opts[b][1]
    return ref_o, ref_l


def check_close(gpu_out, ref_out, gpu_lse=None, ref_lse=None, what="",
                out_max=OUT_MAX, out_mean=OUT_MEAN, lse_max=LSE_MAX, rel_l2=None):
    err = np.abs(gpu_out - ref_out)
    msg = f"{what}: max|d|={err.max():.3e} mean|d|={err.mean():.3e}"
    assert np.isfinite(gpu_out).all(), what + ": non-finite output"
    assert err.max() <= out_max, msg
    assert err.mean() <= out_mean, msg
    if rel_l2 is not None:
        r = np.linalg.norm(gpu_out - ref_out) / max(np.linalg.norm(ref_out), 1e-30)
        assert r <= rel_l2, f"{what}: relative L2 {r:.3e}"
    if gpu_lse is not None:
        le = np.abs(gpu_lse - ref_lse)
        assert le.max() <= lse_max, f"{what}: lse max|d|={le.max():.3e}"
    return err.max(), err.mean()


# the forward computes its row statistics in moment form from this many key
# blocks on (direct form below)
MOMENT_MIN_BLOCKS = 128


def route_mask(sa, q, k, v, B, beta):
    """The GPU's selection mask ``[H, N, nb]`` (numpy bool) under the row
    statistics the sparse forward routes with for these shapes."""
    import torch
    H, N, _ = q.shape
    Nk = k.shape[1]
    kbar, _ = sa.sol_attn_pool(k, v, B)
    if (Nk + B - 1) // B >= MOMENT_MIN_BLOCKS:
        mu, sigma = sa.sol_attn_row_stats_moment(q, kbar, B, Nk)
    else:
        mu, sigma = sa.sol_attn_row_stats(q, kbar, B, Nk)
    m, _ = sa.sol_attn_block_mask(q, kbar, mu, sigma, beta, B, Nk)
    torch.cuda.synchronize()
    return m.cpu().numpy().astype(bool)


def mask_mismatch_ok(gpu_mask, info, beta, eps=TIE_EPS):
    """Masks agree except on pairs the oracle itself calls near-ties."""
    ref = info["mask"]
    diff = np.nonzero(gpu_mask.astype(bool) != ref)
    if len(diff[0]) == 0:
        return True, 0
    tau = info["mu"] + beta * info["sigma"]
    gap = np.abs(info["p"][diff] - tau[diff[0]])
    return bool((gap < eps).all()), len(diff[0])

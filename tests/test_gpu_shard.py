"""GPU parity of key-sharded Sol-Attn on one GPU: each rank's share
(``sol_attn_forward_shard`` over whole key blocks, thresholds from the pooled
keys of every block) against the oracle's key-share mode, and the exact merge
of the shares (``sol_attn_combine_partials``) against the oracle's unsplit
answer.

[DAI] "LTX-2.5 at 4K, in half the time", section "Attention across two GPUs":
the keys are split along the sequence and the partial answers merge exactly.
Here the shares run one after another on the one GPU; the exchange between
ranks is not part of this library.

A share's partial is compared as its part of the whole answer: numerator and
denominator over the unsplit denominator (both bounded), so a share whose own
denominator is small or negative (rejected blocks only) is still checked.
Rows with a near-tie pair are checked through the merged answer only, where
either decision is accepted.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import block_sparse_attention_06_amd as sa  # noqa: E402
import oracle as O  # noqa: E402
from synth import WORKLOADS, clustered, clustered_head, gaussian  # noqa: E402
from tests.parity_utils import (best_match, check_close, dev, host,  # noqa: E402
                                sparse_with_ties, tiles_rows)

pytestmark = pytest.mark.gpu

LN2 = float(np.log(2.0))


def _clustered_small(H, n, B, centres, seed):
    Q = np.empty((H, n, 128), np.uint16)
    K, V = np.empty_like(Q), np.empty_like(Q)
    for h in range(H):
        Q[h], K[h], V[h] = clustered_head(n, 128, B, centres, 0.5, seed, h)
    return Q, K, V


def _run_shares(q, k, v, B, beta, shares):
    """shares: block ranges (b0, b1); returns (part_o [S,H,N,d], part_ml [S,H,N,2],
    merged out, merged lse)."""
    H, N, d = q.shape
    Nk = k.shape[1]
    S = len(shares)
    kbar_all = sa.sol_attn_pool(k, v, B)[0] if beta != float("-inf") else None
    part_o = torch.empty((S, H, N, d), dtype=torch.float32, device=q.device)
    part_ml = torch.empty((S, H, N, 2), dtype=torch.float32, device=q.device)
    for s, (b0, b1) in enumerate(shares):
        ks = k[:, b0 * B:min(Nk, b1 * B)].contiguous()
        vs = v[:, b0 * B:min(Nk, b1 * B)].contiguous()
        sa.sol_attn_forward_shard(q, ks, vs, kbar_all, B=B, beta=beta, part_o=part_o[s],
                                  part_ml=part_ml[s])
    out, lse = sa.sol_attn_combine_partials(part_o, part_ml)
    torch.cuda.synchronize()
    return part_o, part_ml, out, lse


def _check(Q, K, V, B, beta, shares, rows=None, heads=None, what=""):
    q, k, v = dev(Q), dev(K), dev(V)
    H, N, _ = Q.shape
    nb = (K.shape[1] + B - 1) // B
    part_o, part_ml, out, lse = _run_shares(q, k, v, B, beta, shares)
    rows = np.arange(N) if rows is None else rows
    heads = list(range(H)) if heads is None else list(heads)
    # only the sampled heads and rows come back to the host: [heads, rows, ...]
    hi = torch.tensor(heads, device=q.device)
    ri = torch.tensor(rows, device=q.device)
    go, gl = host(out[hi][:, ri]), host(lse[hi][:, ri])
    po, pml = host(part_o[:, hi][:, :, ri]), host(part_ml[:, hi][:, :, ri])
    for a, h in enumerate(heads):
        qh, kh, vh = (O.bf16_to_f64(x[h]) for x in (Q, K, V))
        if beta == float("-inf"):
            o, l = O.dense_head_ref(qh, kh, vh, rows=rows)
            check_close(go[a], o, gl[a], l, what=f"{what} dense merged h{h}")
            tie_free = np.ones(len(rows), bool)
        else:
            o, l, info, cands = sparse_with_ties(qh, kh, vh, B, beta, rows)
            ro, rl = best_match(go[a], gl[a], o, l, cands)
            check_close(go[a], ro, gl[a], rl, what=f"{what} beta {beta} merged h{h}")
            tie_free = np.ones(len(rows), bool)
            tie_free[list(cands)] = False
        # each share's part of the whole answer (rows without near-ties)
        r_ok = rows[tie_free]
        for s, (b0, b1) in enumerate(shares):
            blocks = list(range(b0, min(b1, nb)))
            _, _, inf_s = O.sol_attn_head_ref(qh, kh, vh, B, beta, rows=r_ok, blocks=blocks)
            num, den, M = inf_s["partial"]
            scale = np.exp(M - l[tie_free])
            g_scale = np.exp(pml[s, a, tie_free, 0] * LN2 - l[tie_free])
            g_num = po[s, a, tie_free] * g_scale[:, None]
            g_den = pml[s, a, tie_free, 1] * g_scale
            check_close(g_num, num * scale[:, None], what=f"{what} beta {beta} share {s} h{h}")
            assert np.abs(g_den - den * scale).max() <= 1e-3, f"{what} share {s} h{h}: denominator"


@pytest.mark.parametrize("beta", [0.0, 0.5, 1.0])
def test_shares_clustered_ragged(beta):
    """16 blocks of 64 (the last holds 40 keys), two and three ranks."""
    Q, K, V = _clustered_small(2, 1000, 64, 16, seed=7)
    _check(Q, K, V, 64, beta, [(0, 6), (6, 16)], what="2 ranks")
    _check(Q, K, V, 64, beta, [(0, 3), (3, 10), (10, 16)], what="3 ranks")


@pytest.mark.parametrize("beta", [0.0, 0.5])
def test_shares_unclustered_taylor_heavy(beta):
    """Unclustered inputs: rejected blocks carry a large share of the mass, and
    a share can hold rejected blocks only."""
    Q, K, V = gaussian(2, 640, 128, seed=12)
    _check(Q, K, V, 64, beta, [(0, 4), (4, 10)], what="unclustered")
    _check(Q, K, V, 64, beta, [(0, 1), (1, 9), (9, 10)], what="unclustered 1-block shares")


def test_shares_moment_statistics():
    """129 blocks of 64 over the whole sequence: the thresholds come from the
    moment form of the statistics, computed from every rank's pooled keys."""
    Q, K, V = _clustered_small(2, 129 * 64 - 17, 64, 64, seed=8)
    rows = tiles_rows(Q.shape[1])
    _check(Q, K, V, 64, 0.5, [(0, 64), (64, 129)], rows=rows, what="moments")


def test_shares_dense():
    """beta = -inf: each share is dense attention over its keys."""
    Q, K, V = _clustered_small(2, 1000, 64, 16, seed=9)
    _check(Q, K, V, 64, float("-inf"), [(0, 5), (5, 16)], what="dense")


def test_shares_4k_two_ranks():
    """The 4K workload (H=32, N=130,686, B=128) over two ranks' shares of
    510 and 511 blocks, at full size; sampled tiles of heads 0 and 31; the
    merged answer also against the unsplit call."""
    torch.cuda.empty_cache()
    w = WORKLOADS["4k"]
    Q, K, V = clustered(w, heads=None, threads=16)
    rows = tiles_rows(w.n)
    _check(Q, K, V, w.block, 0.5, [(0, 510), (510, 1021)], rows=rows, heads=(0, 31), what="4k")
    q, k, v = dev(Q), dev(K), dev(V)
    _, _, om, lm = _run_shares(q, k, v, w.block, 0.5, [(0, 510), (510, 1021)])
    ou, lu = sa.sol_attn_forward(q, k, v, B=w.block, beta=0.5)
    torch.cuda.synchronize()
    d = (om.float() - ou.float()).abs()
    assert d.max().item() <= 1e-2 and d.mean().item() <= 1e-4
    assert (lm - lu).abs().max().item() <= 1e-3

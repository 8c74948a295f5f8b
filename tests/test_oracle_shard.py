"""Pins of the oracle's key-share mode (``blocks=``): one rank's partial answer
when the keys are split along the sequence over ranks.

[DAI] "LTX-2.5 at 4K, in half the time", section "Attention across two GPUs":
each GPU attends to its part of the keys and the partial answers, carrying
their running maximum and sum of exponentials, merge exactly.  [SOL] "Stage 2
Optimization -- Core Technology: Sol-Attn": the threshold of a row comes from
the proxy statistics of the whole sequence, so every share uses the same
mu_i, sigma_i; both the exact part and the Taylor part of the method are sums
over key blocks, so the shares' numerators and denominators add up to the
unsplit ones.
"""
import math

import numpy as np
import pytest

import oracle as O


def _rand(rng, n, d, scale=1.0):
    return rng.standard_normal((n, d)) * scale


def _brute_share(q, k, v, B, beta, share):
    """Pure-Python loops: one share's partial (out, lse) for every row."""
    nq, d, nk = len(q), len(q[0]), len(k)
    nb = (nk + B - 1) // B
    s = 1.0 / math.sqrt(d)
    blocks = [list(range(j * B, min(nk, (j + 1) * B))) for j in range(nb)]
    kbar = [[sum(k[t][c] for t in blk) / len(blk) for c in range(d)] for blk in blocks]
    vbar = [[sum(v[t][c] for t in blk) / len(blk) for c in range(d)] for blk in blocks]
    outs, lses = [], []
    for i in range(nq):
        p = [s * sum(q[i][c] * kbar[j][c] for c in range(d)) for j in range(nb)]
        mu = sum(p) / nb
        sigma = math.sqrt(sum((x - mu) ** 2 for x in p) / nb)
        tau = -math.inf if beta == -math.inf else mu + beta * sigma
        num = [0.0] * d
        den = 0.0
        for j in share:
            if p[j] >= tau:
                for t in blocks[j]:
                    e = math.exp(s * sum(q[i][c] * k[t][c] for c in range(d)))
                    den += e
                    for c in range(d):
                        num[c] += e * v[t][c]
            else:
                w = len(blocks[j]) * math.exp(mu) * (1.0 + p[j] - mu)
                den += w
                for c in range(d):
                    num[c] += w * vbar[j][c]
        # a share of rejected blocks alone can have a non-positive denominator
        outs.append([x / den if den > 0 else math.nan for x in num])
        lses.append(math.log(den) if den > 0 else math.nan)
    return np.array(outs), np.array(lses)


@pytest.mark.parametrize("beta", [0.0, 0.5, 1.0, -0.3])
def test_share_matches_brute_force(rng, beta):
    q, k, v = _rand(rng, 6, 8, 1.5), _rand(rng, 45, 8, 1.5), _rand(rng, 45, 8)
    B = 8  # 6 blocks, the last one ragged (5 keys)
    finite = 0
    for share in ([0, 1], [2, 3, 4, 5], [5], [1, 3]):
        o, l, _ = O.sol_attn_head_ref(q, k, v, B, beta, blocks=share)
        bo, bl = _brute_share(q.tolist(), k.tolist(), v.tolist(), B, beta, share)
        ok = np.isfinite(bl)
        np.testing.assert_array_equal(np.isfinite(l), ok)
        np.testing.assert_allclose(o[ok], bo[ok], atol=1e-10)
        np.testing.assert_allclose(l[ok], bl[ok], atol=1e-10)
        finite += int(ok.sum())
    assert finite >= 16, "most (row, share) partials should have a positive denominator"


@pytest.mark.parametrize("beta", [0.0, 0.5, 1.0])
def test_shares_merge_to_the_unsplit_answer(rng, beta):
    """Signed partial sums of shares covering every block once reproduce the
    unsplit result (which the other pins fix against brute force)."""
    q, k, v = _rand(rng, 9, 16, 1.5), _rand(rng, 101, 16, 1.5), _rand(rng, 101, 16)
    B = 16  # 7 blocks, the last one ragged
    o, l, _ = O.sol_attn_head_ref(q, k, v, B, beta)
    for shares in ([[0, 1, 2], [3, 4, 5, 6]], [[0], [1, 2], [3, 4], [5, 6]], [[6], [0, 1, 2, 3, 4, 5]]):
        parts = [O.sol_attn_head_ref(q, k, v, B, beta, blocks=sh)[2]["partial"] for sh in shares]
        M = np.max([pm for _, _, pm in parts], axis=0)
        num = sum(pn * np.exp(pm - M)[:, None] for pn, _, pm in parts)
        den = sum(pd * np.exp(pm - M) for _, pd, pm in parts)
        np.testing.assert_allclose(num / den[:, None], o, atol=1e-12)
        np.testing.assert_allclose(M + np.log(den), l, atol=1e-12)


def test_dense_share_is_attention_over_its_keys(rng):
    """beta = -inf: a share's partial is plain softmax attention over the
    share's keys (library special case: the oracle's dense attention)."""
    q, k, v = _rand(rng, 7, 16), _rand(rng, 70, 16), _rand(rng, 70, 16)
    B = 16
    o, l, _ = O.sol_attn_head_ref(q, k, v, B, -np.inf, blocks=[1, 2])
    do, dl = O.dense_head_ref(q, k[16:48], v[16:48])
    np.testing.assert_allclose(o, do, atol=1e-12)
    np.testing.assert_allclose(l, dl, atol=1e-12)


def test_share_of_rejected_blocks_can_have_a_negative_denominator():
    """A share holding only rejected blocks whose proxy lies more than 1 below
    the row mean has a negative (Taylor-only) denominator: its (out, lse) form
    is undefined (NaN), yet its signed partial still merges exactly."""
    d, B = 2, 2
    q = np.array([[4.0, 0.0]])
    # block 0 far above the mean (selected), block 1 at the mean, block 2 far below
    k = np.array([[6.0, 0.0], [6.0, 0.0], [0.0, 1.0], [0.0, -1.0], [-6.0, 0.0], [-6.0, 0.0]])
    v = np.arange(12, dtype=np.float64).reshape(6, 2)
    o, l, info = O.sol_attn_head_ref(q, k, v, B, 0.5)
    assert info["mask"][0].tolist() == [True, False, False]
    ot, lt, it = O.sol_attn_head_ref(q, k, v, B, 0.5, blocks=[2])
    assert it["partial"][1][0] < 0 and np.isnan(lt[0]) and np.isnan(ot[0]).all()
    parts = [O.sol_attn_head_ref(q, k, v, B, 0.5, blocks=sh)[2]["partial"] for sh in ([0, 1], [2])]
    M = max(p[2][0] for p in parts)
    num = sum(p[0][0] * np.exp(p[2][0] - M) for p in parts)
    den = sum(p[1][0] * np.exp(p[2][0] - M) for p in parts)
    np.testing.assert_allclose(num / den, o[0], atol=1e-12)
    np.testing.assert_allclose(M + np.log(den), l[0], atol=1e-12)


# --------------------------------------------------------------------------
# planted mistakes: each mutated share computation must fail a pin above
# --------------------------------------------------------------------------


def _mutant_share(kind, q, k, v, B, beta, share):
    """One share's partial (out, lse) with one plausible mistake planted."""
    nk, d = k.shape
    nb = (nk + B - 1) // B
    bounds = [(j * B, min(nk, (j + 1) * B)) for j in range(nb)]
    kbar = np.stack([k[s:e].mean(0) for s, e in bounds])
    vbar = np.stack([v[s:e].mean(0) for s, e in bounds])
    p = q @ kbar.T / np.sqrt(d)
    in_share = np.zeros(nb, bool)
    in_share[share] = True
    ps = p[:, in_share] if kind == "stats_from_share" else p
    mu, sigma = ps.mean(1), ps.std(1)
    sel = p >= (mu + beta * sigma)[:, None]
    s = q @ k.T / np.sqrt(d)
    num = np.zeros((q.shape[0], d))
    den = np.zeros(q.shape[0])
    for j, (b0, b1) in enumerate(bounds):
        exact_here = in_share[j] or kind == "exact_all_blocks"
        taylor_here = in_share[j] or kind == "taylor_all_blocks"
        e = np.exp(s[:, b0:b1]) * (sel[:, j:j + 1] & exact_here)
        num += e @ v[b0:b1]
        den += e.sum(1)
        w = np.where(sel[:, j] | (not taylor_here), 0.0,
                     (b1 - b0) * np.exp(mu) * (1 + p[:, j] - mu))
        num += w[:, None] * vbar[j]
        den += w
    with np.errstate(invalid="ignore", divide="ignore"):
        return num / den[:, None], np.where(den > 0, np.log(np.where(den > 0, den, 1.0)), np.nan)


@pytest.mark.parametrize("kind", ["taylor_all_blocks", "stats_from_share", "exact_all_blocks"])
def test_planted_share_mistakes_are_caught(rng, kind):
    q, k, v = _rand(rng, 6, 8, 1.5), _rand(rng, 45, 8, 1.5), _rand(rng, 45, 8)
    failures = 0
    for beta in (0.0, 0.5):
        for share in ([0, 1], [2, 3, 4, 5]):
            o, l = _mutant_share(kind, q, k, v, 8, beta, share)
            bo, bl = _brute_share(q.tolist(), k.tolist(), v.tolist(), 8, beta, share)
            ok = np.isfinite(bl) & np.isfinite(l)
            failures += not (np.allclose(o[ok], bo[ok], atol=1e-10) and
                             np.allclose(l[ok], bl[ok], atol=1e-10) and
                             np.array_equal(np.isfinite(l), np.isfinite(bl)))
    assert failures > 0, f"planted mistake {kind!r} passed every pin"


def test_unmutated_share_copy_passes(rng):
    q, k, v = _rand(rng, 6, 8, 1.5), _rand(rng, 45, 8, 1.5), _rand(rng, 45, 8)
    for share in ([0, 1], [2, 3, 4, 5]):
        o, l = _mutant_share("none", q, k, v, 8, 0.5, share)
        ro, rl, _ = O.sol_attn_head_ref(q, k, v, 8, 0.5, blocks=share)
        ok = np.isfinite(rl)
        np.testing.assert_allclose(o[ok], ro[ok], atol=1e-10)
        np.testing.assert_allclose(l[ok], rl[ok], atol=1e-10)

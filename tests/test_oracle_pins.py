"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each test ties one step to something fixed outside the oracle's code: brute
force on tiny inputs, a library special case, a closed form of the exponential,
an algebraic identity, or an invariance of softmax attention.  A plausible
slip (a dropped term, a wrong sign, B in place of the valid count, sample std,
strict threshold, missing scale, transposed operand) fails at least one test;
``test_planted_mistakes_are_caught`` checks that claim on mutated copies.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from synth import bf16_bits_to_f32, clustered_head, gaussian

# --------------------------------------------------------------------------
# independent brute-force implementations (pure Python, tiny sizes only)
# --------------------------------------------------------------------------


def _dot(a, b):
    return sum(x * y for x, y in zip(a, b))


def brute_dense(q, k, v):
    """Softmax attention from its definition, with Python floats."""
    d = len(q[0])
    outs, lses = [], []
    for qi in q:
        s = [_dot(qi, kt) / math.sqrt(d) for kt in k]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        z = sum(e)
        outs.append([sum(e[t] * v[t][c] for t in range(len(k))) / z for c in range(d)])
        lses.append(m + math.log(z))
    return np.array(outs), np.array(lses)


def brute_sparse(q, k, v, B, beta):
    """The thresholded block-sparse method from its verbal definition, loops only."""
    d = len(q[0])
    nk = len(k)
    blocks = [list(range(s, min(nk, s + B))) for s in range(0, nk, B)]
    kbar = [[sum(k[t][c] for t in blk) / len(blk) for c in range(d)] for blk in blocks]
    vbar = [[sum(v[t][c] for t in blk) / len(blk) for c in range(d)] for blk in blocks]
    outs, lses, masks = [], [], []
    for qi in q:
        p = [_dot(qi, kb) / math.sqrt(d) for kb in kbar]
        mu = sum(p) / len(p)
        sigma = math.sqrt(sum((x - mu) ** 2 for x in p) / len(p))
        if beta == -math.inf:
            sel = [True] * len(p)
        elif beta == math.inf:
            sel = [False] * len(p)
        else:
            sel = [x >= mu + beta * sigma for x in p]
        num = [0.0] * d
        den = 0.0
        for j, blk in enumerate(blocks):
            if sel[j]:
                for t in blk:
                    w = math.exp(_dot(qi, k[t]) / math.sqrt(d))
                    den += w
                    for c in range(d):
                        num[c] += w * v[t][c]
            else:
                w = len(blk) * math.exp(mu) * (1.0 + p[j] - mu)
                den += w
                for c in range(d):
                    num[c] += w * vbar[j][c]
        outs.append([x / den for x in num])
        lses.append(math.log(den))
        masks.append(sel)
    return np.array(outs), np.array(lses), np.array(masks)


def _rand(rng, n, d, scale=1.0):
    return rng.standard_normal((n, d)) * scale


# --------------------------------------------------------------------------
# dense path
# --------------------------------------------------------------------------


@pytest.mark.parametrize("n,nk,d", [(1, 1, 4), (5, 5, 4), (3, 13, 8), (7, 64, 4)])
def test_dense_matches_bruteforce(n, nk, d, rng):
    q, k, v = _rand(rng, n, d, 2.0), _rand(rng, nk, d, 2.0), _rand(rng, nk, d)
    o, l = O.dense_head_ref(q, k, v)
    ob, lb = brute_dense(q.tolist(), k.tolist(), v.tolist())
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, lb, rtol=0, atol=1e-12)


def test_dense_matches_torch_sdpa_fp64(rng):
    """Library special case: PyTorch's CPU scaled_dot_product_attention in fp64."""
    q, k, v = _rand(rng, 70, 128), _rand(rng, 130, 128), _rand(rng, 130, 128)
    o, l = O.dense_head_ref(q, k, v)
    t = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None])
    np.testing.assert_allclose(o, t[0].numpy(), rtol=0, atol=1e-12)
    # lse against torch.logsumexp of the scaled logits
    s = torch.from_numpy(q) @ torch.from_numpy(k).T / math.sqrt(128)
    np.testing.assert_allclose(l, torch.logsumexp(s, dim=1).numpy(), rtol=0, atol=1e-12)


def test_dense_ragged_equals_masked_padding(rng):
    """A ragged key set equals the padded set with the pad keys masked to -inf
    (doubleAI, "Attention across two GPUs": dropping the pad gives the same result)."""
    q, k, v = _rand(rng, 9, 16), _rand(rng, 130, 16), _rand(rng, 130, 16)
    o, l = O.dense_head_ref(q, k, v)
    kp = np.concatenate([k, _rand(rng, 2, 16)])
    vp = np.concatenate([v, _rand(rng, 2, 16)])
    mask = torch.zeros(9, 132, dtype=torch.float64)
    mask[:, 130:] = -math.inf
    t = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(kp)[None], torch.from_numpy(vp)[None],
        attn_mask=mask[None])
    np.testing.assert_allclose(o, t[0].numpy(), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# sparse path: brute force and identities
# --------------------------------------------------------------------------


@pytest.mark.parametrize("nk,B,beta", [(16, 4, 0.0), (18, 4, 0.5), (13, 4, 1.0),
                                       (20, 5, -0.3), (12, 4, float("inf"))])
def test_sparse_matches_bruteforce(nk, B, beta, rng):
    q, k, v = _rand(rng, 6, 4, 1.5), _rand(rng, nk, 4, 1.5), _rand(rng, nk, 4)
    o, l, info = O.sol_attn_head_ref(q, k, v, B, beta)
    ob, lb, mb = brute_sparse(q.tolist(), k.tolist(), v.tolist(), B, beta)
    np.testing.assert_array_equal(info["mask"], mb)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-11)
    np.testing.assert_allclose(l, lb, rtol=0, atol=1e-11)


def test_beta_neg_inf_is_dense(rng):
    q, k, v = _rand(rng, 40, 32), _rand(rng, 150, 32), _rand(rng, 150, 32)
    o, l, info = O.sol_attn_head_ref(q, k, v, 16, float("-inf"))
    od, ld = O.dense_head_ref(q, k, v)
    assert info["mask"].all()
    np.testing.assert_allclose(o, od, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l, ld, rtol=0, atol=1e-12)


def test_all_blocks_selected_has_no_taylor_term(rng):
    """A finite beta low enough that tau_i < min_j p_ij selects every block; the
    result must then be the plain dense result (no Taylor mass anywhere)."""
    q, k, v = _rand(rng, 40, 32), _rand(rng, 150, 32), _rand(rng, 150, 32)
    o, l, info = O.sol_attn_head_ref(q, k, v, 16, -1e6)
    od, ld = O.dense_head_ref(q, k, v)
    assert info["mask"].all()
    np.testing.assert_allclose(o, od, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l, ld, rtol=0, atol=1e-12)


def test_split_merge_equals_unsplit(rng):
    """Partial answers over two halves of the keys merge exactly (doubleAI,
    "Attention across two GPUs")."""
    q, k, v = _rand(rng, 12, 128), _rand(rng, 1000, 128), _rand(rng, 1000, 128)
    o, l = O.dense_head_ref(q, k, v)
    oa, la = O.dense_head_ref(q, k[:613], v[:613])
    ob, lb = O.dense_head_ref(q, k[613:], v[613:])
    om, lm = O.lse_merge_ref(oa, la, ob, lb)
    np.testing.assert_allclose(om, o, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lm, l, rtol=0, atol=1e-13)


def test_merge_edge_cases():
    out_a = np.array([[1.0, 2.0], [3.0, 4.0]])
    out_b = np.array([[5.0, 6.0], [7.0, 8.0]])
    lse_a = np.array([-np.inf, 0.0])
    lse_b = np.array([-np.inf, -np.inf])
    om, lm = O.lse_merge_ref(out_a, lse_a, out_b, lse_b)
    np.testing.assert_array_equal(om[0], [0.0, 0.0])
    assert np.isneginf(lm[0])
    np.testing.assert_array_equal(om[1], out_a[1])
    assert lm[1] == 0.0
    # equal masses: plain average, lse + log 2
    om, lm = O.lse_merge_ref(out_a, np.zeros(2), out_b, np.zeros(2))
    np.testing.assert_allclose(om, (out_a + out_b) / 2)
    np.testing.assert_allclose(lm, np.log(2.0))


def test_sparse_split_over_key_blocks_merges_exactly(rng):
    """Both the exact and the Taylor parts are sums over key blocks, so sparse
    partials over whole-block halves of the keys merge like dense partials, when
    both halves use the full-sequence statistics.  The oracle has no split mode,
    so this checks the decomposition the split kernel relies on: the merged
    numerators and denominators reproduce the unsplit result."""
    q, k, v = _rand(rng, 8, 16, 1.5), _rand(rng, 96, 16, 1.5), _rand(rng, 96, 16)
    B = 8
    o, l, info = O.sol_attn_head_ref(q, k, v, B, 0.25)
    # rebuild per-block masses from the definition and split them in two halves
    sel, p, mu = info["mask"], info["p"], info["mu"]
    vbar = O.pool_ref(v, B)
    s = q @ k.T / 4.0
    num = np.zeros((2, 8, 16))
    den = np.zeros((2, 8))
    for j in range(12):
        half = 0 if j < 5 else 1
        if (sel[:, j]).any():
            e = np.exp(s[:, j * B:(j + 1) * B]) * sel[:, j:j + 1]
            num[half] += e @ v[j * B:(j + 1) * B]
            den[half] += e.sum(1)
        w = np.where(sel[:, j], 0.0, B * np.exp(mu) * (1 + p[:, j] - mu))
        num[half] += w[:, None] * vbar[j]
        den[half] += w
    np.testing.assert_allclose((num[0] + num[1]) / (den[0] + den[1])[:, None], o, atol=1e-12)
    np.testing.assert_allclose(np.log(den[0] + den[1]), l, atol=1e-12)


# --------------------------------------------------------------------------
# pooling, proxy and statistics
# --------------------------------------------------------------------------


def test_pool_is_block_mean_ragged():
    x = np.arange(10 * 3, dtype=np.float64).reshape(10, 3)
    kb = O.pool_ref(x, 4)
    np.testing.assert_array_equal(kb[0], x[0:4].sum(0) / 4)
    np.testing.assert_array_equal(kb[1], x[4:8].sum(0) / 4)
    np.testing.assert_array_equal(kb[2], x[8:10].sum(0) / 2)   # ragged: 2 valid tokens


def test_proxy_is_mean_of_block_logits(rng):
    """p_ij equals the mean over the block of the exact scaled logits (linearity)."""
    q, k = _rand(rng, 11, 64), _rand(rng, 203, 64)
    p = O.proxy_ref(q, O.pool_ref(k, 32))
    s = np.einsum("id,td->it", q, k) / 8.0
    mean_s = np.stack([s[:, a:b].mean(1) for a, b in O.block_bounds(203, 32)], axis=1)
    np.testing.assert_allclose(p, mean_s, rtol=0, atol=3e-14)


def test_stats_bruteforce_and_moment_form(rng):
    """Row statistics against a loop, and against the moment form
    mu = s q.mean(kbar), sigma^2 = s^2 q^T Cov(kbar) q (population covariance)."""
    q, k = _rand(rng, 9, 32), _rand(rng, 300, 32)
    kbar = O.pool_ref(k, 16)
    p = O.proxy_ref(q, kbar)
    mu, sigma = O.row_stats_ref(p)
    for i in range(9):
        row = p[i].tolist()
        m = sum(row) / len(row)
        sd = math.sqrt(sum((x - m) ** 2 for x in row) / len(row))
        assert abs(mu[i] - m) < 1e-13 and abs(sigma[i] - sd) < 1e-13
    sc = 1 / math.sqrt(32)
    cov = np.cov(kbar.T, bias=True)
    np.testing.assert_allclose(mu, sc * q @ kbar.mean(0), atol=1e-13)
    np.testing.assert_allclose(sigma ** 2, sc * sc * np.einsum("id,de,ie->i", q, cov, q),
                               atol=1e-12)


def test_selection_threshold_semantics():
    p = np.array([[1.0, 2.0, 3.0, 4.0],
                  [5.0, 5.0, 5.0, 5.0]])
    mu, sigma = O.row_stats_ref(p)
    assert sigma[1] == 0.0
    # "at or above": a row whose blocks all equal the threshold selects them all
    for beta in (0.0, 0.5, 3.0):
        assert O.select_ref(p, mu, sigma, beta)[1].all()
    # beta = 0: tau = mu = 2.5 -> blocks 3 and 4
    np.testing.assert_array_equal(O.select_ref(p, mu, sigma, 0.0)[0], [0, 0, 1, 1])
    assert O.select_ref(p, mu, sigma, float("-inf")).all()
    assert not O.select_ref(p, mu, sigma, float("inf")).any()
    # an exact tie at a finite beta: p = (0, 0, 3, 3) has mu = sigma = 1.5, tau(1) = 3
    p2 = np.array([[0.0, 0.0, 3.0, 3.0]])
    m2, s2 = O.row_stats_ref(p2)
    np.testing.assert_array_equal(O.select_ref(p2, m2, s2, 1.0)[0], [0, 0, 1, 1])


def test_selection_monotone_in_beta(rng):
    q, k = _rand(rng, 50, 32), _rand(rng, 640, 32)
    p = O.proxy_ref(q, O.pool_ref(k, 32))
    mu, sigma = O.row_stats_ref(p)
    prev = O.select_ref(p, mu, sigma, -2.0)
    for beta in (-1.0, -0.2, 0.0, 0.3, 0.5, 1.0, 2.0):
        cur = O.select_ref(p, mu, sigma, beta)
        assert not (cur & ~prev).any()          # nested
        prev = cur


def test_near_ties_listed():
    p = np.array([[0.0, 1.0, 2.00000001]])
    mu, sigma = O.row_stats_ref(p)
    ties = O.near_ties_ref(p, mu, sigma, (2.0 - mu[0]) / sigma[0], 1e-4)
    assert ties == [(0, 2)]


# --------------------------------------------------------------------------
# the Taylor term: closed form on constant blocks
# --------------------------------------------------------------------------


def _constant_blocks(levels, sizes, d=4, x=1.0):
    """Keys all equal inside a block, values all equal inside a block; the only
    nonzero key coordinate gives logits s_t = levels[j] * x for the block."""
    q = np.zeros((1, d))
    q[0, 0] = x
    ks, vs = [], []
    rng = np.random.default_rng(7)
    vals = rng.standard_normal((len(levels), d))
    for j, (lev, n) in enumerate(zip(levels, sizes)):
        kj = np.zeros(d)
        kj[0] = lev * math.sqrt(d)
        ks.append(np.tile(kj, (n, 1)))
        vs.append(np.tile(vals[j], (n, 1)))
    return q, np.concatenate(ks), np.concatenate(vs), vals


@pytest.mark.parametrize("levels,beta", [((-1.0, 0.0, 1.0), 0.5),
                                         ((-0.7, 0.2, 1.3, 0.1), 0.0),
                                         ((0.5, -1.5, 2.0, 0.4), 0.9)])
def test_taylor_closed_form_on_constant_blocks(levels, beta):
    """For a block whose tokens share one key and one value, its exact mass is
    n e^{p} and the first-order term about mu is n e^{mu} (1 + p - mu); the
    sparse result must differ from dense by exactly n e^{mu}(e^{d} - 1 - d),
    d = p - mu, in the denominator (and that times v in the numerator), for
    each rejected block.  The last block is ragged (3 tokens) to pin n_j."""
    B = 8
    sizes = [B] * (len(levels) - 1) + [3]
    q, k, v, vals = _constant_blocks(levels, sizes)
    o, l, info = O.sol_attn_head_ref(q, k, v, B, beta)
    p = np.array(levels, dtype=np.float64)
    mu = p.mean()
    sd = math.sqrt(((p - mu) ** 2).mean())
    sel = p >= mu + beta * sd
    np.testing.assert_array_equal(info["mask"][0], sel)
    assert (~sel).any() and sel.any()
    n = np.array(sizes, dtype=np.float64)
    num_dense = (n * np.exp(p)) @ vals
    den_dense = (n * np.exp(p)).sum()
    dlt = p - mu
    gap = np.where(sel, 0.0, n * math.exp(mu) * (np.exp(dlt) - 1 - dlt))
    num = num_dense - gap @ vals
    den = den_dense - gap.sum()
    np.testing.assert_allclose(o[0], num / den, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l[0], math.log(den), rtol=0, atol=1e-13)


def test_taylor_exact_when_rejected_block_sits_at_mean():
    """A constant block with p_ij = mu_i is reproduced exactly by the Taylor term."""
    q, k, v, vals = _constant_blocks((-1.0, 0.0, 1.0), (8, 8, 8))
    o, l, info = O.sol_attn_head_ref(q, k, v, 8, 0.5)
    np.testing.assert_array_equal(info["mask"][0], [False, False, True])
    # block 0 has 1 + p - mu = 0: zero weight; block 1 is exact
    num = 8 * math.e * vals[2] + 8 * 1.0 * vals[1]
    den = 8 * math.e + 8
    np.testing.assert_allclose(o[0], num / den, rtol=0, atol=1e-14)


# --------------------------------------------------------------------------
# invariances
# --------------------------------------------------------------------------


def _clustered_small(seed=3, n=192, d=32, B=16):
    q, k, v = clustered_head(n, d, B, 6, 0.5, seed, 0)
    return (bf16_bits_to_f32(q).astype(np.float64), bf16_bits_to_f32(k).astype(np.float64),
            bf16_bits_to_f32(v).astype(np.float64))


def test_invariance_block_permutation():
    q, k, v = _clustered_small()
    B = 16
    o, l, _ = O.sol_attn_head_ref(q, k, v, B, 0.3)
    perm = np.random.default_rng(0).permutation(k.shape[0] // B)
    idx = np.concatenate([np.arange(j * B, (j + 1) * B) for j in perm])
    o2, l2, _ = O.sol_attn_head_ref(q, k[idx], v[idx], B, 0.3)
    np.testing.assert_allclose(o2, o, atol=1e-13)
    np.testing.assert_allclose(l2, l, atol=1e-12)


def test_invariance_token_permutation_within_blocks():
    q, k, v = _clustered_small()
    B = 16
    o, l, _ = O.sol_attn_head_ref(q, k, v, B, 0.5)
    rng = np.random.default_rng(1)
    idx = np.concatenate([j * B + rng.permutation(B) for j in range(k.shape[0] // B)])
    o2, l2, _ = O.sol_attn_head_ref(q, k[idx], v[idx], B, 0.5)
    np.testing.assert_allclose(o2, o, atol=1e-13)
    np.testing.assert_allclose(l2, l, atol=1e-12)


def test_invariance_value_shift():
    """Every weight multiplies a value and enters the denominator, so V + c -> out + c."""
    q, k, v = _clustered_small()
    o, l, _ = O.sol_attn_head_ref(q, k, v, 16, 0.5)
    c = np.linspace(-1, 1, v.shape[1])
    o2, l2, _ = O.sol_attn_head_ref(q, k, v + c, 16, 0.5)
    np.testing.assert_allclose(o2, o + c, atol=1e-12)
    np.testing.assert_allclose(l2, l, atol=1e-13)


def test_invariance_key_shift():
    """k_t + c for all t shifts every logit of row i by q_i.c/sqrt(d): selection is
    unchanged, out is unchanged and lse moves by that shift."""
    q, k, v = _clustered_small()
    c = np.random.default_rng(5).standard_normal(k.shape[1]) * 0.3
    o, l, info = O.sol_attn_head_ref(q, k, v, 16, 0.5)
    o2, l2, info2 = O.sol_attn_head_ref(q, k + c, v, 16, 0.5)
    np.testing.assert_array_equal(info["mask"], info2["mask"])
    np.testing.assert_allclose(o2, o, atol=1e-12)
    np.testing.assert_allclose(l2, l + q @ c / math.sqrt(k.shape[1]), atol=1e-12)


def test_rows_subset_matches_full():
    q, k, v = _clustered_small()
    o, l, _ = O.sol_attn_head_ref(q, k, v, 16, 0.5)
    rows = [0, 5, 100, 191]
    o2, l2, _ = O.sol_attn_head_ref(q, k, v, 16, 0.5, rows=rows)
    np.testing.assert_array_equal(o2, o[rows])
    np.testing.assert_array_equal(l2, l[rows])


# --------------------------------------------------------------------------
# quality (not parity): the Taylor term recovers mass hard selection drops
# --------------------------------------------------------------------------


def test_taylor_recovers_mass_vs_hard_selection():
    Q, K, V = gaussian(1, 256, 64, seed=11)
    q, k, v = (bf16_bits_to_f32(x[0]).astype(np.float64) for x in (Q, K, V))
    od, _ = O.dense_head_ref(q, k, v)
    ot, _, _ = O.sol_attn_head_ref(q, k, v, 16, 0.5)
    oh, _, _ = O.sol_attn_head_ref(q, k, v, 16, 0.5, taylor=False)
    assert np.abs(ot - od).max() < np.abs(oh - od).max()


# --------------------------------------------------------------------------
# the pins above catch planted mistakes (mutated copies of the oracle, on the CPU)
# --------------------------------------------------------------------------


def _mutant_forward(kind):
    """A copy of the sparse forward with one plausible mistake planted."""
    def f(q, k, v, B, beta):
        nq, d = q.shape
        nk = k.shape[0]
        bounds = O.block_bounds(nk, B)
        n_j = np.array([e - s for s, e in bounds], dtype=np.float64)
        if kind == "B_for_nj":
            n_j = np.full_like(n_j, B)
        kbar, vbar = O.pool_ref(k, B), O.pool_ref(v, B)
        scale = 1 / math.sqrt(d)
        if kind == "no_scale_proxy":
            p = q @ kbar.T
        else:
            p = O.proxy_ref(q, kbar)
        mu = p.mean(1)
        if kind == "sample_std":
            sigma = p.std(1, ddof=1)
        else:
            sigma = p.std(1)
        tau = mu + beta * sigma
        sel = p > tau[:, None] if kind == "strict" else p >= tau[:, None]
        tb = np.repeat(np.arange(len(bounds)), n_j.astype(np.int64) if kind != "B_for_nj"
                       else np.array([e - s for s, e in bounds]))
        s = scale * q @ k.T
        e = np.where(sel[:, tb], np.exp(s), 0.0)
        num, den = e @ v, e.sum(1)
        sign = -1.0 if kind == "wrong_sign" else 1.0
        w = np.where(sel, 0.0, n_j * np.exp(mu)[:, None] * (1 + sign * (p - mu[:, None])))
        if kind != "no_taylor_num":
            num = num + w @ vbar
        den = den + w.sum(1)
        return num / den[:, None], np.log(den)
    return f


@pytest.mark.parametrize("kind", ["B_for_nj", "no_scale_proxy", "sample_std", "strict",
                                  "wrong_sign", "no_taylor_num"])
def test_planted_mistakes_are_caught(kind):
    """Each mutant must fail at least one of the independent pins used above."""
    f = _mutant_forward(kind)
    failures = 0
    # constant-block closed form (pins n_j, sign, numerator term)
    for levels, beta in [((-1.0, 0.0, 1.0), 0.5), ((-0.7, 0.2, 1.3, 0.1), 0.0)]:
        B = 8
        sizes = [B] * (len(levels) - 1) + [3]
        q, k, v, vals = _constant_blocks(levels, sizes)
        p = np.array(levels)
        mu, sd = p.mean(), p.std()
        sel = p >= mu + beta * sd
        n = np.array(sizes, dtype=np.float64)
        dl = p - mu
        gap = np.where(sel, 0.0, n * math.exp(mu) * (np.exp(dl) - 1 - dl))
        ref = ((n * np.exp(p)) @ vals - gap @ vals) / ((n * np.exp(p)).sum() - gap.sum())
        o, _ = f(q, k, v, B, beta)
        failures += not np.allclose(o[0], ref, atol=1e-10)
    # brute force on tiny random inputs (pins scale, std, threshold)
    rng = np.random.default_rng(99)
    for nk, B, beta in [(16, 4, 0.0), (18, 4, 0.5), (13, 4, 1.0)]:
        q, k, v = _rand(rng, 6, 4, 1.5), _rand(rng, nk, 4, 1.5), _rand(rng, nk, 4)
        ob, _, _ = brute_sparse(q.tolist(), k.tolist(), v.tolist(), B, beta)
        o, _ = f(q, k, v, B, beta)
        failures += not np.allclose(o, ob, atol=1e-10)
    # value-shift invariance (pins Taylor in both numerator and denominator)
    q, k, v = _clustered_small()
    o1, _ = f(q, k, v, 16, 0.5)
    o2, _ = f(q, k, v + 0.7, 16, 0.5)
    failures += not np.allclose(o2, o1 + 0.7, atol=1e-10)
    # exact ties (pins "at or above")
    q, k, v, vals = _constant_blocks((0.0, 0.0, 3.0, 3.0), (4, 4, 4, 4))
    ob, _, mb = brute_sparse(q.tolist(), k.tolist(), v.tolist(), 4, 1.0)
    o, _ = f(q, k, v, 4, 1.0)
    failures += not np.allclose(o, ob, atol=1e-12)
    assert failures > 0, f"planted mistake {kind!r} passed every pin"


@pytest.mark.parametrize("beta", [0.0, 0.7, float("inf"), -5.0])
def test_zero_spread_closed_form(beta):
    """sigma_i = 0 (all keys equal, so every proxy score equals mu_i and every
    logit equals s_i): the exact part and the Taylor part give the same mass per
    block, so whatever the tied selection, out = mean of V and lse = s + ln(Nk).
    Pins the oracle's sigma = 0 handling (tau = mu for finite beta, nothing
    selected for +inf) and the Taylor weight on a ragged last block (n_j = 5)."""
    rng = np.random.default_rng(8)
    n, nk, d, B = 7, 37, 16, 8
    q = rng.standard_normal((n, d))
    k = np.repeat(rng.standard_normal((1, d)), nk, axis=0)
    v = rng.standard_normal((nk, d))
    out, lse, info = O.sol_attn_head_ref(q, k, v, B, beta)
    # the spread is zero up to the rounding of the fp64 means (every score is a
    # near-tie then, and either decision gives the same answer)
    assert np.all(info["sigma"] < 1e-14)
    s = q @ k[0] / math.sqrt(d)
    np.testing.assert_allclose(out, np.broadcast_to(v.mean(axis=0), out.shape), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, s + math.log(nk), rtol=0, atol=1e-12)
    if beta == float("inf"):
        assert not info["mask"].any()
    # every decision forced the other way: the same answer
    force = {(i, j): not bool(info["mask"][i, j]) for i in range(n) for j in range(info["mask"].shape[1])}
    fo, fl, _ = O.sol_attn_head_ref(q, k, v, B, beta, force=force)
    np.testing.assert_allclose(fo, out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(fl, lse, rtol=0, atol=1e-12)

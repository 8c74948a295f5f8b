"""GPU parity of every C-ABI entry point against the fp64 oracle, at sizes the
oracle finishes in seconds that still span several tiles and a ragged tail.

Tolerances (unit-scale V): out max abs <= 1e-2 and mean abs <= 1e-3; lse max
abs <= 1e-3; selection masks exact except near-ties (|p - tau| < 1e-4 by the
oracle's own scores); pooled means and proxy scores to fp32-level bounds
stated per test.
"""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import block_sparse_attention_06_amd as sa  # noqa: E402
import oracle as O  # noqa: E402
from synth import clustered, clustered_head, gaussian, WORKLOADS  # noqa: E402
from tests.parity_utils import (best_match, check_close, dev, host, mask_mismatch_ok,  # noqa: E402
                                route_mask, sparse_with_ties, tiles_rows)

pytestmark = pytest.mark.gpu

INF = float("inf")


def _head(bits, h):
    return O.bf16_to_f64(bits[h])


def _clustered_small(H, N, B, seed=70):
    """Clustered recipe (one centre per key block, one per query block) at a
    given shape; heads 0..H-1."""
    from synth import Workload
    nb = (N + B - 1) // B
    w = Workload("custom", H, N, 0, 128, B, nb, 0.5, seed, (0.5,))
    return clustered(w)


# ---------------------------------------------------------------------------
# pooling and routing
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("H,N,B", [(2, 2048, 64), (3, 1000, 128), (1, 77, 64), (2, 128, 128)])
def test_pool_parity(H, N, B):
    Q, K, V = gaussian(H, N, 128, seed=40 + N)
    kbar, vbar = sa.sol_attn_pool(dev(K), dev(V), B)
    torch.cuda.synchronize()
    for h in range(H):
        kr = O.pool_ref(_head(K, h), B)
        vr = O.pool_ref(_head(V, h), B)
        # fp32 sum of <= 128 bf16 values, then one division
        np.testing.assert_allclose(host(kbar[h]), kr, rtol=0, atol=2e-6)
        np.testing.assert_allclose(host(vbar[h]), vr, rtol=0, atol=2e-6)


@pytest.mark.parametrize("case", ["tiny_clustered", "gauss_ragged"])
def test_proxy_and_stats_parity(case):
    if case == "tiny_clustered":
        w = WORKLOADS["tiny"]
        Q, K, V = clustered(w)
        B, N = w.block, w.n
    else:
        Q, K, V = gaussian(2, 1500, 128, seed=5)
        B, N = 128, 1500
    q, kk = dev(Q), dev(K)
    kbar, _ = sa.sol_attn_pool(kk, dev(V), B)
    p = sa.sol_attn_proxy_scores(q, kbar, B, N)
    mu, sigma = sa.sol_attn_row_stats(q, kbar, B, N)
    torch.cuda.synchronize()
    for h in range(Q.shape[0]):
        kb = O.pool_ref(_head(K, h), B)
        pr = O.proxy_ref(_head(Q, h), kb)
        mr, sr = O.row_stats_ref(pr)
        # hi/lo split of kbar: ~16 significant bits -> |dp| well below the 1e-4 tie
        # band (measured: proxy 8.2e-6, mu 1.7e-6, sigma 9.7e-6 on the clustered
        # tiny shape, whose scores are the largest here)
        assert np.abs(host(p[h]) - pr).max() < 2e-5
        assert np.abs(host(mu[h]) - mr).max() < 1e-5
        assert np.abs(host(sigma[h]) - sr).max() < 2e-5


@pytest.mark.parametrize("H,N,B", [(2, 2048, 64), (2, 1500, 128), (2, 20000, 128), (1, 130, 64),
                                   (2, 130686, 128), (1, 130686, 64)])
def test_row_stats_moment_parity(H, N, B):
    """Moment form (mean and covariance of the pooled keys) against the oracle's
    statistics of the proxy scores, and against the direct form on the GPU.
    The last two shapes have the 4K workload's block counts (1021 blocks of
    128, 2042 of 64, the last one ragged); there the oracle checks whole
    first, middle and last 128-row tiles."""
    Q, K, V = gaussian(H, N, 128, seed=60 + N + B)
    q = dev(Q)
    kbar, _ = sa.sol_attn_pool(dev(K), dev(V), B)
    mu, sigma = sa.sol_attn_row_stats_moment(q, kbar, B, N)
    mu_d, sigma_d = sa.sol_attn_row_stats(q, kbar, B, N)
    torch.cuda.synchronize()
    rows = np.arange(N) if N <= 20000 else tiles_rows(N)
    for h in range(H):
        kb = O.pool_ref(_head(K, h), B)
        mr, sr = O.row_stats_ref(O.proxy_ref(_head(Q, h)[rows], kb))
        # the moment form computes sigma^2, so a small sigma magnifies its error by
        # 1 / (2 sigma): 1.3e-5 at sigma = 0.013 on the 3-block shape, at most
        # 1e-6 elsewhere (mu: at most 3.2e-7)
        assert np.abs(host(mu[h])[rows] - mr).max() < 1e-5
        assert np.abs(host(sigma[h])[rows] - sr).max() < 2e-5
    assert (mu - mu_d).abs().max().item() < 4e-5
    assert (sigma - sigma_d).abs().max().item() < 4e-5


@pytest.mark.parametrize("beta", [0.0, 0.5, 1.0])
def test_block_mask_parity_moment_form(beta):
    """157 key blocks (ragged last one): the forward call routes with the
    moment-form statistics from 128 blocks on, so the mask is built from
    those, with the forward kernel's own proxy and predicate, and compared
    with the oracle's selection outside the near-tie band."""
    H, N, B = 2, 20000, 128
    Q, K, V = _clustered_small(H, N, B)
    q = dev(Q)
    kbar, _ = sa.sol_attn_pool(dev(K), dev(V), B)
    mu, sigma = sa.sol_attn_row_stats_moment(q, kbar, B, N)
    rows = tiles_rows(N)
    masks = []
    for t0 in sorted(set((rows // 128) * 128)):
        m, _ = sa.sol_attn_block_mask(q, kbar, mu, sigma, beta, B, N, row0=int(t0),
                                      nrows=min(128, N - int(t0)))
        masks.append(m.cpu().numpy())
    torch.cuda.synchronize()
    for h in range(H):
        kb = O.pool_ref(_head(K, h), B)
        p = O.proxy_ref(_head(Q, h)[rows], kb)
        mr, sr = O.row_stats_ref(p)
        info = dict(p=p, mu=mr, sigma=sr, mask=O.select_ref(p, mr, sr, beta))
        gm = np.concatenate([m[h] for m in masks])
        ok, n = mask_mismatch_ok(gm, info, beta)
        assert ok, f"head {h}: {n} mask mismatches outside the near-tie band"


@pytest.mark.parametrize("beta", [0.0, 0.5, 1.0, -0.5])
def test_block_mask_parity(beta):
    w = WORKLOADS["tiny"]
    Q, K, V = clustered(w) if beta != -0.5 else gaussian(2, 2048, 128, seed=8)
    B, N = w.block, w.n
    q = dev(Q)
    kbar, _ = sa.sol_attn_pool(dev(K), dev(V), B)
    mu, sigma = sa.sol_attn_row_stats(q, kbar, B, N)
    mask, counts = sa.sol_attn_block_mask(q, kbar, mu, sigma, beta, B, N)
    torch.cuda.synchronize()
    m = mask.cpu().numpy()
    total_sel = 0
    for h in range(Q.shape[0]):
        kb = O.pool_ref(_head(K, h), B)
        p = O.proxy_ref(_head(Q, h), kb)
        mr, sr = O.row_stats_ref(p)
        info = dict(p=p, mu=mr, sigma=sr, mask=O.select_ref(p, mr, sr, beta))
        ok, n = mask_mismatch_ok(m[h], info, beta)
        assert ok, f"head {h}: {n} mask mismatches outside the near-tie band"
        total_sel += int(m[h].sum())
    c = counts.cpu().numpy()
    assert c[0] == total_sel
    nb = (N + B - 1) // B
    assert c[3] == Q.shape[0] * ((N + 127) // 128) * nb
    assert c[0] <= 32 * c[1] and c[1] <= 4 * c[2] and c[2] <= c[3]


# ---------------------------------------------------------------------------
# forward: dense
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("H,N,Nk", [(2, 2048, 2048), (2, 300, 300), (1, 1, 1), (3, 126, 5000),
                                    (2, 700, 129), (1, 130, 4097)])
def test_dense_forward_parity(H, N, Nk):
    Q, K, V = gaussian(H, N, 128, seed=N + Nk, nk=Nk)
    out, lse = sa.sol_attn_forward(dev(Q), dev(K), dev(V), mode=sa.SOL_DENSE)
    torch.cuda.synchronize()
    for h in range(H):
        o, l = O.dense_head_ref(_head(Q, h), _head(K, h), _head(V, h))
        check_close(host(out[h]), o, host(lse[h]), l, what=f"dense H{H} N{N} Nk{Nk} h{h}")


def test_dense_tiny_clustered():
    w = WORKLOADS["tiny"]
    Q, K, V = clustered(w)
    out, lse = sa.sol_attn_forward(dev(Q), dev(K), dev(V), mode=sa.SOL_DENSE)
    torch.cuda.synchronize()
    o, l = O.dense_ref(Q, K, V)
    check_close(host(out), o, host(lse), l, what="dense tiny")


# ---------------------------------------------------------------------------
# forward: sparse
# ---------------------------------------------------------------------------


def _sparse_case(Q, K, V, B, beta, heads=None, rows=None):
    """Sparse forward against the oracle on the given heads and rows.  The GPU's
    own selection (same statistics form as the forward) must match the oracle's
    outside the tie band, and settles rows with more near-ties than the
    enumeration covers."""
    q, k, v = dev(Q), dev(K), dev(V)
    out, lse = sa.sol_attn_forward(q, k, v, B=B, beta=beta, mode=sa.SOL_SPARSE)
    torch.cuda.synchronize()
    go, gl = host(out), host(lse)
    gmask = route_mask(sa, q, k, v, B, beta)
    heads = range(Q.shape[0]) if heads is None else heads
    for h in heads:
        r = np.arange(Q.shape[1]) if rows is None else rows
        o, l, info, cands = sparse_with_ties(_head(Q, h), _head(K, h), _head(V, h), B, beta, r,
                                             gpu_mask=gmask[h][r])
        ok, nbad = mask_mismatch_ok(gmask[h][r], info, beta)
        assert ok, f"sparse B{B} beta{beta} h{h}: {nbad} mask mismatches outside the tie band"
        ro, rl = best_match(go[h][r], gl[h][r], o, l, cands)
        check_close(go[h][r], ro, gl[h][r], rl, what=f"sparse B{B} beta{beta} h{h}")
    return go, gl


@pytest.mark.parametrize("beta", [0.0, float("-inf")])
def test_sparse_tiny_clustered(beta):
    w = WORKLOADS["tiny"]
    Q, K, V = clustered(w)
    _sparse_case(Q, K, V, w.block, beta)


@pytest.mark.parametrize("beta", [0.0, 0.5, 1.0, INF, -0.3])
@pytest.mark.parametrize("B", [64, 128])
def test_sparse_unclustered_taylor_heavy(beta, B):
    """Unclustered N(0,1): the Taylor term carries a large share of the mass."""
    Q, K, V = gaussian(2, 1000, 128, seed=77 + B)
    _sparse_case(Q, K, V, B, beta)


def test_sparse_ragged_and_short_query():
    Q, K, V = gaussian(2, 250, 128, seed=3, nk=1234)
    _sparse_case(Q, K, V, 128, 0.5)
    Q, K, V = gaussian(1, 1, 128, seed=4, nk=200)
    _sparse_case(Q, K, V, 64, 0.0)


@pytest.mark.parametrize("N,Nk,B,beta", [
    (3900, 3900, 128, 0.5),     # last query tile ragged
    (4000, 3037, 64, 0.0),      # keys end inside a 32-key unit
    (3968, 4100, 128, -0.3),    # query tiles end exactly on a tile
    (4096, 4096, 64, INF),      # nothing selected: Taylor terms only
    (3900, 2500, 128, -1e6),    # every block selected
])
def test_sparse_many_tiles(N, Nk, B, beta):
    """Sixteen heads of ~4K rows: enough query tiles to fill the chip without a
    key split, as long sequences run; checked on the first and last head, all
    rows."""
    H = 16
    Q, K, V = gaussian(H, N, 128, seed=N + Nk + B, nk=Nk)
    _sparse_case(Q, K, V, B, beta, heads=(0, H - 1))


def _growing_logits(H, N, Nk, slope, seed):
    """Logits that grow along the keys by about `slope` nats per key (q has a
    component of 4 along dimension 0, key t one of 0.7 * slope / 0.25 * t):
    at 0.25 nats per key every 32-key unit outruns the running reference by
    more than 8 log2 units, so the softmax moves its reference on every unit."""
    from synth import f32_to_bf16_bits
    rng = np.random.default_rng(seed)
    q = 0.3 * rng.standard_normal((H, N, 128)).astype(np.float32)
    k = 0.3 * rng.standard_normal((H, Nk, 128)).astype(np.float32)
    v = rng.standard_normal((H, Nk, 128)).astype(np.float32)
    q[:, :, 0] = 4.0
    k[:, :, 0] = (slope * math.sqrt(128) / 4.0) * np.arange(Nk, dtype=np.float32)
    return f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)


def test_dense_reference_moves_on_every_unit():
    """Dense mode with logits rising ~0.25 nats per key up to ~370: the
    reference of the running sums is moved (and the sums rescaled) on every
    unit, with the keys split over workgroups (short query set), with one
    4-wave workgroup per 128-row query tile, and with the 12-wave form on
    384-row tiles (32 heads x 11 tiles: its last tile holds 100 rows, so waves
    4-11 hold none and wave 3 four; the last 32-key unit is ragged).

    A handful of keys carry the mass here, so a denominator summed from the
    bf16-rounded probabilities would be off by up to 2^-9 relative in ln(l)
    (about 2e-3); the kernels sum the fp32 probabilities, and lse keeps the
    1e-3 bound of every other case."""
    # split keys / 4-wave tiles (512) / 12-wave tiles (352, ragged last tile)
    for H, N in ((2, 200), (16, 4096), (32, 3940)):
        Q, K, V = _growing_logits(H, N, 1500, 0.25, seed=N)
        out, lse = sa.sol_attn_forward(dev(Q), dev(K), dev(V), mode=sa.SOL_DENSE)
        torch.cuda.synchronize()
        rows = np.union1d(np.arange(0, N, max(1, N // 200)), np.arange(max(0, N - 130), N))
        for h in (0, H - 1):
            o, l = O.dense_head_ref(_head(Q, h), _head(K, h), _head(V, h), rows=rows)
            check_close(host(out[h])[rows], o, host(lse[h])[rows], l, what=f"dense growing N{N} h{h}")


@pytest.mark.parametrize("B", [64, 128])
def test_sparse_reference_moves_on_every_unit(B):
    """Sparse mode on the same rising logits: the reference starts at mu, far
    below the selected blocks' scores, and moves on every selected unit; the
    rejected early blocks' Taylor weights are negligible next to e^max.  lse
    within 1e-3, as in the dense case (fp32 denominator)."""
    Q, K, V = _growing_logits(2, 300, 1500, 0.25, seed=B)  # keys split over workgroups
    _sparse_case(Q, K, V, B, 0.0)
    Q, K, V = _growing_logits(16, 4096, 1500, 0.25, seed=B + 1)  # one workgroup per tile
    _sparse_case(Q, K, V, B, 0.0, heads=(0, 15), rows=np.arange(0, 4096, 17))


def test_sparse_split_keys_short_query():
    """Few query tiles: the sparse key range is split over workgroups (chunks of
    32 blocks) and merged; must match the unsplit oracle."""
    Q, K, V = gaussian(2, 100, 128, seed=9, nk=64 * 200)
    _sparse_case(Q, K, V, 64, 0.5)


def test_sparse_neg_inf_is_dense_bitwise():
    w = WORKLOADS["tiny"]
    Q, K, V = clustered(w)
    q, k, v = dev(Q), dev(K), dev(V)
    o1, l1 = sa.sol_attn_forward(q, k, v, B=64, beta=float("-inf"), mode=sa.SOL_SPARSE)
    o2, l2 = sa.sol_attn_forward(q, k, v, mode=sa.SOL_DENSE)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_all_blocks_selected_matches_dense_oracle():
    Q, K, V = gaussian(2, 700, 128, seed=12)
    out, lse = sa.sol_attn_forward(dev(Q), dev(K), dev(V), B=128, beta=-1e6, mode=sa.SOL_SPARSE)
    torch.cuda.synchronize()
    for h in range(2):
        o, l = O.dense_head_ref(_head(Q, h), _head(K, h), _head(V, h))
        check_close(host(out[h]), o, host(lse[h]), l, what="all-selected")


def test_forward_deterministic():
    w = WORKLOADS["tiny"]
    Q, K, V = clustered(w)
    q, k, v = dev(Q), dev(K), dev(V)
    a = sa.sol_attn_forward(q, k, v, B=64, beta=0.0)
    b = sa.sol_attn_forward(q, k, v, B=64, beta=0.0)
    c = sa.sol_attn_forward(q, k, v, mode=sa.SOL_DENSE)
    d = sa.sol_attn_forward(q, k, v, mode=sa.SOL_DENSE)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert torch.equal(c[0], d[0]) and torch.equal(c[1], d[1])


# ---------------------------------------------------------------------------
# LSE merge
# ---------------------------------------------------------------------------


def test_lse_merge_parity_and_edges():
    Q, K, V = gaussian(2, 126, 128, seed=21, nk=3000)
    q, k, v = dev(Q), dev(K), dev(V)
    oa, la = sa.sol_attn_forward(q, k[:, :1700].contiguous(), v[:, :1700].contiguous(),
                                 mode=sa.SOL_DENSE)
    ob, lb = sa.sol_attn_forward(q, k[:, 1700:].contiguous(), v[:, 1700:].contiguous(),
                                 mode=sa.SOL_DENSE)
    om, lm = sa.attn_lse_merge(oa, la, ob, lb)
    torch.cuda.synchronize()
    for h in range(2):
        o, l = O.dense_head_ref(_head(Q, h), _head(K, h), _head(V, h))
        check_close(host(om[h]), o, host(lm[h]), l, what="merge vs unsplit")
        # the merge kernel itself against the oracle merge of the same bf16 inputs
        ro, rl = O.lse_merge_ref(host(oa[h]), host(la[h]), host(ob[h]), host(lb[h]))
        np.testing.assert_allclose(host(om[h]), ro, rtol=0, atol=4e-3 * np.abs(ro).max() + 1e-6)
        np.testing.assert_allclose(host(lm[h]), rl, rtol=0, atol=1e-5)
    # edges: both empty -> 0 / -inf; one empty -> the other
    la2 = la.clone()
    la2[0, :3] = -INF
    lb2 = lb.clone()
    lb2[0, :3] = -INF
    lb2[1, :5] = -INF
    om2, lm2 = sa.attn_lse_merge(oa, la2, ob, lb2)
    torch.cuda.synchronize()
    assert torch.all(om2[0, :3] == 0) and torch.all(torch.isneginf(lm2[0, :3]))
    assert torch.equal(om2[1, :5], oa[1, :5]) and torch.equal(lm2[1, :5], la2[1, :5])
    # in place on out_a / lse_a
    oa_c, la_c = oa.clone(), la.clone()
    sa.attn_lse_merge(oa_c, la_c, ob, lb, out=oa_c, lse=la_c)
    torch.cuda.synchronize()
    assert torch.equal(oa_c, om) and torch.equal(la_c, lm)


# ---------------------------------------------------------------------------
# argument errors reported, nothing launched
# ---------------------------------------------------------------------------


def test_error_codes_through_binding():
    q = torch.zeros((1, 64, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(sa.SolAttnError) as e:
        sa.sol_attn_forward(q, q, q, B=32, beta=0.0)
    assert e.value.code == -2
    small_ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(sa.SolAttnError) as e:
        sa.sol_attn_forward(q, q, q, B=64, beta=0.0, workspace=small_ws)
    assert e.value.code == -1


def test_binding_rejects_mis_sized_buffers():
    """Buffers smaller than the sizes passed with them, or a workspace in host
    memory, are refused by the binding before any launch (the C ABI takes
    plain pointers and cannot check them)."""
    H, N = 2, 256
    q = torch.zeros((H, N, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        sa.sol_attn_forward(q, q, q, B=64, beta=0.0, lse=torch.empty((H, N - 1), device="cuda"))
    with pytest.raises(ValueError):
        sa.sol_attn_forward(q, q, q, B=64, beta=0.0,
                            workspace=torch.empty(1 << 20, dtype=torch.uint8))
    lse = torch.zeros((H, N), device="cuda")
    with pytest.raises(ValueError):
        sa.attn_lse_merge(q, lse, q[:, :128].contiguous(), lse)
    with pytest.raises(ValueError):
        sa.attn_lse_merge(q, lse, q, lse, out=torch.empty_like(q)[:1].contiguous())
    kbar, _ = sa.sol_attn_pool(q, q, 64)
    with pytest.raises(ValueError):
        sa.sol_attn_row_stats(q, kbar[:, :-1].contiguous(), 64, N)
    with pytest.raises(ValueError):
        sa.sol_attn_proxy_scores(q, kbar, 64, N, row0=200, nrows=100)
    with pytest.raises(ValueError):
        sa.sol_attn_pool(q, q[:, :100].contiguous(), 64)
    # correctly sized buffers still work
    out, l2 = sa.sol_attn_forward(q, q, q, B=64, beta=0.0, lse=torch.empty((H, N), device="cuda"))
    torch.cuda.synchronize()
    assert torch.isfinite(l2).all()


# ---------------------------------------------------------------------------
# degenerate statistics: zero spread
# ---------------------------------------------------------------------------


def _zero_spread(case, H=2, N=300, Nk=1000):
    """bf16 bits of (Q, K, V) with sigma_i = 0 for every row: every key equal
    (``same_keys``) or every query zero (``zero_queries``); 1000 keys in blocks
    of 64 leave a ragged last block of 40."""
    from synth import f32_to_bf16_bits
    rng = np.random.default_rng(77)
    q = rng.standard_normal((H, N, 128)).astype(np.float32)
    v = rng.standard_normal((H, Nk, 128)).astype(np.float32)
    if case == "same_keys":
        k = np.repeat(0.2 * rng.standard_normal((H, 1, 128)).astype(np.float32), Nk, axis=1)
    else:
        k = rng.standard_normal((H, Nk, 128)).astype(np.float32)
        q[:] = 0.0
    return f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)


@pytest.mark.parametrize("beta", [0.0, 0.5, INF, -1e6])
@pytest.mark.parametrize("case", ["same_keys", "zero_queries"])
def test_zero_spread_closed_form(case, beta):
    """sigma_i = 0: every proxy score equals mu_i, so every block ties with the
    threshold and either decision is allowed.  Every key of a row then has the
    same logit s_i = p_ij = mu_i, and a rejected block's Taylor weight
    n_j e^{mu}(1 + p - mu) = n_j e^{s} equals its exact softmax mass, with the
    block's value sum: whatever the selection, out = mean of V and
    lse = s_i + ln(Nk).  Also one query row against one key."""
    Q, K, V = _zero_spread(case)
    out, lse = sa.sol_attn_forward(dev(Q), dev(K), dev(V), B=64, beta=beta, mode=sa.SOL_SPARSE)
    torch.cuda.synchronize()
    go, gl = host(out), host(lse)
    for h in range(Q.shape[0]):
        q, k, v = _head(Q, h), _head(K, h), _head(V, h)
        s = (q @ k[0]) / math.sqrt(128)
        check_close(go[h], np.broadcast_to(v.mean(axis=0), go[h].shape), gl[h],
                    s + math.log(k.shape[0]), what=f"{case} beta {beta} h{h}")
    q1, k1, v1 = (x[:1, :1].copy() for x in (Q, K, V))
    o1, l1 = sa.sol_attn_forward(dev(q1), dev(k1), dev(v1), B=64, beta=beta, mode=sa.SOL_SPARSE)
    torch.cuda.synchronize()
    s1 = float(_head(q1, 0)[0] @ _head(k1, 0)[0]) / math.sqrt(128)
    check_close(host(o1[0]), _head(v1, 0), host(l1[0]), np.array([s1]), what=f"{case} 1x1 beta {beta}")

"""CPU checks of the parity helpers' near-tie handling (no GPU).

The tie band follows the stated mask tolerance: pairs with |p - tau| below
1e-4 may be decided either way, so the reference for such a row is any of the
oracle's answers under the possible decisions.  These tests widen the band on
purpose so that every row has several "near-tie" pairs, and check the two ways
the helper builds the reference: enumeration up to the cap, and the GPU's own
decisions beyond it.
"""
import numpy as np
import pytest

import oracle as O
from tests.parity_utils import best_match, mask_mismatch_ok, sparse_with_ties


def _case(seed=5, n=96, nk=256, B=64):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((n, 128))
    k = rng.standard_normal((nk, 128))
    v = rng.standard_normal((nk, 128))
    return q, k, v, B


def test_enumeration_holds_the_oracle_answer():
    q, k, v, B = _case()
    rows = np.arange(0, 96, 7)
    # a wide band: most rows get two or three "ties" among 4 blocks
    out, lse, info, cands = sparse_with_ties(q, k, v, B, 0.5, rows, eps=0.5, max_ties=4)
    assert cands, "the widened band must create near-tie rows"
    for i, opts in cands.items():
        n_ties = int(np.log2(len(opts)))
        assert len(opts) == 2 ** n_ties
        # the oracle's own decisions are one of the candidates
        assert any(np.array_equal(o, out[i]) and l == lse[i] for o, l in opts)
    # the reference picked for the oracle's own answer is that answer
    ro, rl = best_match(out, lse, out, lse, cands)
    np.testing.assert_array_equal(ro, out)
    np.testing.assert_array_equal(rl, lse)


def test_rows_beyond_the_cap_take_the_gpu_decisions():
    q, k, v, B = _case()
    rows = np.arange(0, 96, 5)
    # every block a "tie", cap 1: every row with a tie goes past the cap
    with pytest.raises(AssertionError, match="enumeration cap"):
        sparse_with_ties(q, k, v, B, 0.5, rows, eps=1e9, max_ties=1)
    out, lse, info = O.sol_attn_head_ref(q, k, v, B, 0.5, rows=rows)
    # GPU decisions equal to the oracle's: the single candidate is the oracle answer
    _, _, _, cands = sparse_with_ties(q, k, v, B, 0.5, rows, eps=1e9, max_ties=1,
                                      gpu_mask=info["mask"])
    for i, opts in cands.items():
        assert len(opts) == 1
        np.testing.assert_allclose(opts[0][0], out[i], rtol=0, atol=1e-12)
        np.testing.assert_allclose(opts[0][1], lse[i], rtol=0, atol=1e-12)
    # GPU decisions flipped on every pair: the candidate is the oracle under that mask
    flipped = ~info["mask"]
    _, _, _, cands = sparse_with_ties(q, k, v, B, 0.5, rows, eps=1e9, max_ties=1,
                                      gpu_mask=flipped)
    force = {(int(r), j): bool(flipped[i][j]) for i, r in enumerate(rows)
             for j in range(flipped.shape[1])}
    fo, fl, _ = O.sol_attn_head_ref(q, k, v, B, 0.5, rows=rows, force=force)
    for i, opts in cands.items():
        np.testing.assert_allclose(opts[0][0], fo[i], rtol=0, atol=1e-12)
        np.testing.assert_allclose(opts[0][1], fl[i], rtol=0, atol=1e-12)


def test_mask_mismatch_only_inside_the_band():
    q, k, v, B = _case()
    rows = np.arange(0, 96, 3)
    _, _, info = O.sol_attn_head_ref(q, k, v, B, 0.5, rows=rows)
    ok, n = mask_mismatch_ok(info["mask"], info, 0.5)
    assert ok and n == 0
    # flip the pair closest to its threshold: inside a band that wide, outside 1e-4
    tau = info["mu"] + 0.5 * info["sigma"]
    gap = np.abs(info["p"] - tau[:, None])
    i, j = np.unravel_index(np.argmin(gap), gap.shape)
    bad = info["mask"].copy()
    bad[i, j] = not bad[i, j]
    ok, n = mask_mismatch_ok(bad, info, 0.5, eps=gap[i, j] * 2)
    assert ok and n == 1
    ok, n = mask_mismatch_ok(bad, info, 0.5, eps=gap[i, j] / 2)
    assert not ok and n == 1

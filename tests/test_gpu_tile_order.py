"""The order in which sparse forward calls run their 128-row query tiles
(sol_attn_tile_schedule, and the forward call itself):

- the per-tile work counts equal the 128-row unions of the selection mask the
  inspection call reports, up to the blocks whose decision for the tile's most
  selective row lies within the rounding of the count's proxy (it uses the
  bf16 high part of the pooled keys only): at most 3 blocks per tile, 0.5 on
  average;
- the order is, per head, a stable sort of the tiles by decreasing count;
- the order decides only when a tile runs: a four-head call that orders its
  2,048 tiles equals, bit for bit, the four single-head calls of 512 tiles,
  which run in natural order (neither splits its keys), and every output row
  is written; likewise with a ragged last tile (4 heads of 65,636 rows);
- at beta = +inf (no block selected) and beta = -1e6 (every block selected)
  all tiles carry the same work and run in natural order.

Inputs: the clustered generator (one centre per 128-row query block), seeded."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import block_sparse_attention_06_amd as sa  # noqa: E402
from synth import Workload, clustered  # noqa: E402
from tests.parity_utils import dev  # noqa: E402

pytestmark = pytest.mark.gpu


def _inputs(H, N, seed, B=128):
    w = Workload("order", H, N, 0, 128, B, (N + B - 1) // B, 0.5, seed, (0.5,))
    Q, K, V = clustered(w, threads=16)
    return dev(Q), dev(K), dev(V)


@pytest.mark.parametrize("H,N,B,beta", [(4, 40000, 128, 0.5), (2, 20000, 64, 1.0),
                                        (3, 3000, 128, 0.0)])
def test_schedule_counts_and_order(H, N, B, beta):
    q, k, v = _inputs(H, N, seed=41 + H)
    work, order = sa.sol_attn_tile_schedule(q, k, v, B=B, beta=beta)
    n_qt = (N + 127) // 128
    nb = (N + B - 1) // B
    # the selection the call routes with: moment-form statistics from 128 blocks on
    kbar, _ = sa.sol_attn_pool(k, v, B)
    if nb >= 128:
        mu, sigma = sa.sol_attn_row_stats_moment(q, kbar, B, N)
    else:
        mu, sigma = sa.sol_attn_row_stats(q, kbar, B, N)
    mask, _ = sa.sol_attn_block_mask(q, kbar, mu, sigma, beta, B, N)
    pad = n_qt * 128 - N
    m = torch.nn.functional.pad(mask, (0, 0, 0, pad)).bool()
    union = m.view(H, n_qt, 128, nb).any(dim=2).sum(-1).to(torch.int32)
    torch.cuda.synchronize()
    w, u, o = work.cpu().numpy(), union.cpu().numpy(), order.cpu().numpy()
    diff = np.abs(w - u)
    # a tile's union changes when the proxy of its most selective row for a block
    # sits within the high part's rounding of the threshold: measured on about
    # 15 % of the tiles at 313 blocks, by one or two blocks of about 235
    assert diff.max() <= 3, f"work counts off the mask's unions by up to {diff.max()}"
    assert diff.mean() <= 0.5, f"mean difference {diff.mean():.3f} blocks"
    for h in range(H):
        want = h * n_qt + np.lexsort((np.arange(n_qt), -w[h]))  # decreasing work, then index
        np.testing.assert_array_equal(o[h * n_qt:(h + 1) * n_qt], want, err_msg=f"head {h}")


@pytest.mark.parametrize("H,N,B,beta", [(4, 65536, 128, 0.5), (4, 65536, 64, 1.0),
                                        (4, 65636, 128, 0.5)])
def test_ordered_call_equals_natural_order_calls(H, N, B, beta):
    # 4 x 512 tiles, or 4 x 513 with a ragged last tile of 100 rows: the call
    # orders its tiles; one head alone has too few tiles to order, and enough
    # not to split its keys (512 workgroups or more)
    q, k, v = _inputs(H, N, seed=47, B=B)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((H, N), float("nan"), dtype=torch.float32, device="cuda")
    sa.sol_attn_forward(q, k, v, B=B, beta=beta, out=out, lse=lse)
    work, order = sa.sol_attn_tile_schedule(q, k, v, B=B, beta=beta)
    torch.cuda.synchronize()
    assert not torch.isnan(out.float()).any() and not torch.isnan(lse).any(), "a row was not written"
    n_qt = (N + 127) // 128
    o = order.cpu().numpy()
    assert not np.array_equal(o, np.arange(H * n_qt)), "the call should run its tiles out of natural order"
    for h in range(H):
        oh, lh = sa.sol_attn_forward(q[h:h + 1].contiguous(), k[h:h + 1].contiguous(),
                                     v[h:h + 1].contiguous(), B=B, beta=beta)
        torch.cuda.synchronize()
        assert torch.equal(oh[0], out[h]), f"head {h}: output differs from the single-head call"
        assert torch.equal(lh[0], lse[h]), f"head {h}: lse differs from the single-head call"


@pytest.mark.parametrize("beta,count", [(float("inf"), "none"), (-1e6, "all")])
def test_degenerate_beta_counts_and_natural_order(beta, count):
    """beta = +inf selects no block (Taylor terms only) and beta = -1e6 every block:
    every tile then carries the same work (0 or all blocks, the ragged last
    block included), the order is the natural one, and the ordered call still
    equals the single-head calls bit for bit."""
    H, N, B = 4, 65536, 128
    q, k, v = _inputs(H, N, seed=59, B=B)
    work, order = sa.sol_attn_tile_schedule(q, k, v, B=B, beta=beta)
    out, lse = sa.sol_attn_forward(q, k, v, B=B, beta=beta)
    torch.cuda.synchronize()
    n_qt, nb = N // 128, N // B
    want = 0 if count == "none" else nb
    assert (work.cpu().numpy() == want).all(), f"work counts should all be {want}"
    np.testing.assert_array_equal(order.cpu().numpy(), np.arange(H * n_qt))
    for h in (0, H - 1):
        oh, lh = sa.sol_attn_forward(q[h:h + 1].contiguous(), k[h:h + 1].contiguous(),
                                     v[h:h + 1].contiguous(), B=B, beta=beta)
        torch.cuda.synchronize()
        assert torch.equal(oh[0], out[h]) and torch.equal(lh[0], lse[h]), f"head {h}"


def test_schedule_argument_errors():
    q, k, v = _inputs(1, 1000, seed=53)
    with pytest.raises(sa.SolAttnError):
        sa.sol_attn_tile_schedule(q, k, v, B=128, beta=float("-inf"))
    with pytest.raises(sa.SolAttnError):
        sa.sol_attn_tile_schedule(q, k, v, B=96, beta=0.5)

"""GPU parity of ``na3d_forward`` (3D neighbourhood attention) against
``oracle.na3d``: grids with ragged patches along every axis (frame groups of
four, 4 x 8 query patches), windows from 1 x 3 x 5 to the widest column
window (25), both unit shapes (2 x 16 keys up to kx = 9, 1 x 32 beyond), the
whole grid, and the 4K decoder-tile shape on sampled rows.  Tolerances as
for the attention kernels: out max abs <= 1e-2, mean abs <= 1e-3, lse max
abs <= 1e-3."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import block_sparse_attention_06_amd as sa  # noqa: E402
import oracle.na3d as NA  # noqa: E402
from synth import gaussian  # noqa: E402
from tests.parity_utils import check_close, dev, host  # noqa: E402

pytestmark = pytest.mark.gpu


def _case(H, grid, window, seed, heads=None, rows=None):
    n = int(np.prod(grid))
    Q, K, V = gaussian(H, n, 128, seed=seed)
    out, lse = sa.na3d_forward(dev(Q), dev(K), dev(V), grid, window)
    torch.cuda.synchronize()
    heads = list(range(H)) if heads is None else heads
    ro, rl = NA.na3d_ref(Q, K, V, grid, window, heads=heads, rows=rows)
    go, gl = host(out), host(lse)
    for i, h in enumerate(heads):
        r = slice(None) if rows is None else rows
        check_close(go[h][r], ro[i], gl[h][r], rl[i], what=f"na3d {grid} {window} h{h}")


@pytest.mark.parametrize("grid,window", [
    ((2, 9, 20), (1, 3, 5)),      # ragged row band (1 row) and column brick (4 columns)
    ((4, 17, 37), (3, 7, 7)),
    ((3, 8, 20), (3, 7, 17)),
    ((4, 12, 40), (3, 11, 9)),
    ((2, 6, 7), (1, 5, 7)),       # fewer than 32 columns
    ((3, 5, 15), (3, 5, 15)),     # the window is the whole grid: dense attention
    ((5, 9, 33), (5, 3, 25)),     # widest column window; a frame group with one frame
    ((6, 10, 26), (3, 5, 11)),    # first window on 1 x 32 units
    ((7, 13, 30), (3, 9, 9)),     # last window on 2 x 16 units; ragged frame group
    ((1, 4, 9), (1, 3, 9)),       # one frame
    ((9, 6, 12), (7, 5, 11)),
    ((3, 1, 20), (1, 1, 5)),      # one row: 1 x 32 units
    ((2, 3, 10), (1, 3, 7)),      # odd row count: the last row group moves up one row
])
def test_na3d_parity(grid, window):
    _case(2, grid, window, seed=sum(grid) + sum(window))


def test_na3d_decoder_tile_sampled():
    """Four frames of the 4K latent grid (68 x 120), window 3 x 7 x 7, 16 heads;
    rows sampled over the grid's corners, edges and interior."""
    grid, window = (4, 68, 120), (3, 7, 7)
    n = int(np.prod(grid))
    rows = np.unique(np.concatenate([np.arange(0, n, 997), [0, 119, 120 * 67, n - 1, n - 120]]))
    _case(16, grid, window, seed=11, heads=[0, 15], rows=rows)


def test_na3d_argument_errors():
    q = torch.zeros((1, 2 * 4 * 4, 128), dtype=torch.bfloat16, device="cuda")
    for window in [(2, 3, 3), (1, 5, 3), (1, 3, 0)]:
        with pytest.raises(sa.SolAttnError):
            sa.na3d_forward(q, q, q, (2, 4, 4), window)
    q = torch.zeros((1, 1 * 2 * 27, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(sa.SolAttnError):  # wider than 25 columns: unsupported
        sa.na3d_forward(q, q, q, (1, 2, 27), (1, 1, 27))

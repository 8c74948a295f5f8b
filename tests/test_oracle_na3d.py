"""Pins of the 3D neighbourhood-attention oracle (``oracle.na3d``): window
placement by hand-worked cases and by an independent rule (the k grid
positions nearest the query), the full-grid window against torch's fp64
attention, and brute force on a tiny grid.  CPU only."""
import numpy as np
import pytest

import oracle.na3d as NA

torch = pytest.importorskip("torch")


def test_window_start_cases():
    # axis of length 10, window 3: centred inside, shifted inward at the ends
    assert [NA.window_start(p, 10, 3) for p in (0, 1, 2, 5, 8, 9)] == [0, 0, 1, 4, 7, 7]
    # window 7 on an axis of 9
    assert [NA.window_start(p, 9, 7) for p in range(9)] == [0, 0, 0, 0, 1, 2, 2, 2, 2]
    assert all(NA.window_start(p, 5, 5) == 0 for p in range(5))
    with pytest.raises(ValueError):
        NA.window_start(0, 10, 4)
    with pytest.raises(ValueError):
        NA.window_start(0, 3, 5)


def test_window_is_the_k_nearest_positions():
    """For odd k the shifted window is exactly the set of the k positions
    closest to p (an independent characterisation)."""
    for L in range(1, 14):
        for k in range(1, L + 1, 2):
            for p in range(L):
                order = sorted(range(L), key=lambda j: (abs(j - p), j))
                nearest = set(order[:k])
                s = NA.window_start(p, L, k)
                assert set(range(s, s + k)) == nearest, (L, k, p)


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_full_grid_window_is_dense_attention():
    grid, d = (3, 5, 7), 16  # odd extents: the window may span the whole grid
    n = int(np.prod(grid))
    q, k, v = _rand((n, d), 1), _rand((n, d), 2), _rand((n, d), 3)
    out, lse = NA.na3d_head_ref(q, k, v, grid, grid)
    tq, tk, tv = (torch.from_numpy(a)[None, None] for a in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)[0, 0].numpy()
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    s = (q @ k.T) / np.sqrt(d)
    np.testing.assert_allclose(lse, np.log(np.exp(s).sum(axis=1)), rtol=0, atol=1e-12)


def _brute(q, k, v, grid, window):
    """Loops only: each query's window is the set of grid points whose
    coordinates are among the k nearest on every axis (ties toward the lower
    index), softmax with scale 1/sqrt(d) over it."""
    T, Y, X = grid
    n, d = q.shape

    def nearest(p, L, kk):
        return set(sorted(range(L), key=lambda j: (abs(j - p), j))[:kk])

    outs, lses = [], []
    for i in range(n):
        t, y, x = i // (Y * X), (i // X) % Y, i % X
        keys = [j for j in range(n)
                if j // (Y * X) in nearest(t, T, window[0])
                and (j // X) % Y in nearest(y, Y, window[1])
                and j % X in nearest(x, X, window[2])]
        assert len(keys) == np.prod(window)
        w = [np.exp(sum(q[i, c] * k[j, c] for c in range(d)) / np.sqrt(d)) for j in keys]
        outs.append(sum(wj * v[j] for wj, j in zip(w, keys)) / sum(w))
        lses.append(np.log(sum(w)))
    return np.array(outs), np.array(lses)


def test_brute_force_tiny_grid():
    grid, window, d = (3, 5, 6), (3, 3, 5), 8
    n = int(np.prod(grid))
    q, k, v = _rand((n, d), 4), _rand((n, d), 5), _rand((n, d), 6)
    out, lse = NA.na3d_head_ref(q, k, v, grid, window)
    bo, bl = _brute(q, k, v, grid, window)
    np.testing.assert_allclose(out, bo, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, bl, rtol=1e-12, atol=1e-12)


def test_constant_values_and_row_subsets():
    grid, window, d = (4, 6, 7), (3, 5, 5), 8
    n = int(np.prod(grid))
    q, k = _rand((n, d), 7), _rand((n, d), 8)
    v = np.full((n, d), 0.75)
    out, _ = NA.na3d_head_ref(q, k, v, grid, window)
    np.testing.assert_allclose(out, 0.75, rtol=0, atol=1e-14)
    v = _rand((n, d), 9)
    full, lf = NA.na3d_head_ref(q, k, v, grid, window)
    rows = [0, 17, n - 1]
    part, lp = NA.na3d_head_ref(q, k, v, grid, window, rows=rows)
    assert np.array_equal(part, full[rows]) and np.array_equal(lp, lf[rows])


# --------------------------------------------------------------------------
# planted mistakes: each mutated copy must fail one of the pins above
# --------------------------------------------------------------------------


def _mutant(kind):
    """A copy of the oracle's per-head computation with one plausible mistake."""
    def start(p, L, kk):
        if kind == "no_clamp":
            return max(p - kk // 2, 0)          # not shifted inward at the far end
        if kind == "off_by_one":
            return min(max(p - kk // 2 + 1, 0), L - kk)
        return min(max(p - kk // 2, 0), L - kk)

    def f(q, k, v, grid, window):
        T, Y, X = grid
        kt, ky, kx = window
        n, d = q.shape
        scale = 1.0 if kind == "no_scale" else 1.0 / np.sqrt(d)
        out, lse = np.empty((n, d)), np.empty(n)
        for i in range(n):
            t, y, x = i // (Y * X), (i // X) % Y, i % X
            if kind == "swap_axes":                 # rows and columns exchanged
                y, x = i % Y, (i // Y) % X
            t0, y0, x0 = start(t, T, kt), start(y, Y, ky), start(x, X, kx)
            idx = [(tt * Y + yy) * X + xx for tt in range(t0, min(T, t0 + kt))
                   for yy in range(y0, min(Y, y0 + ky)) for xx in range(x0, min(X, x0 + kx))]
            s = (k[idx] @ q[i]) * scale
            m = s.max()
            e = np.exp(s - m)
            out[i] = (e @ v[idx]) / e.sum()
            lse[i] = m + np.log(e.sum()) if kind != "lse_log2" else (m + np.log(e.sum())) / np.log(2)
        return out, lse
    return f


@pytest.mark.parametrize("kind", ["no_clamp", "off_by_one", "no_scale", "swap_axes", "lse_log2"])
def test_planted_mistakes_are_caught(kind):
    f = _mutant(kind)
    failures = 0
    grid, window, d = (3, 5, 6), (3, 3, 5), 8
    n = int(np.prod(grid))
    q, k, v = _rand((n, d), 4), _rand((n, d), 5), _rand((n, d), 6)
    bo, bl = _brute(q, k, v, grid, window)
    o, l = f(q, k, v, grid, window)
    failures += not (np.allclose(o, bo, atol=1e-10) and np.allclose(l, bl, atol=1e-10))
    grid = (3, 5, 7)
    n = int(np.prod(grid))
    q, k, v = _rand((n, 16), 1), _rand((n, 16), 2), _rand((n, 16), 3)
    tq, tk, tv = (torch.from_numpy(a)[None, None] for a in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)[0, 0].numpy()
    o, _ = f(q, k, v, grid, grid)
    failures += not np.allclose(o, ref, atol=1e-10)
    assert failures > 0, f"planted mistake {kind!r} passed every pin"


def test_unmutated_copy_passes_the_pins():
    """The mutant harness itself, without a mistake, agrees with the oracle."""
    f = _mutant("none")
    grid, window, d = (3, 5, 6), (3, 3, 5), 8
    n = int(np.prod(grid))
    q, k, v = _rand((n, d), 4), _rand((n, d), 5), _rand((n, d), 6)
    o, l = f(q, k, v, grid, window)
    ro, rl = NA.na3d_head_ref(q, k, v, grid, window)
    np.testing.assert_allclose(o, ro, atol=1e-12)
    np.testing.assert_allclose(l, rl, atol=1e-12)

"""fp64 CPU oracle for 3D neighbourhood attention over a video token grid.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this module: only the test suite and the ``cpu_baseline`` leg of ``bench.py``
use it.  It shares no code, header, table or helper with the HIP library.

Source: [DAI] "LTX-2.5 at 4K, in half the time" (doubleAI), section "Inside
the decoder": the diffusion video decoder spends most of its time in one
neighbourhood-attention kernel over tiles of four frames; and the LTX-2
pipelines optimization guide (mirror), which names the 3D neighbourhood
attention (na3d) backends of that decoder.

Readings where the pages are silent (each also listed in the design notes):

* tokens lie on a (T, Y, X) grid, flattened frame-major then row-major;
* a query at (t, y, x) attends to the kt x ky x kx keys of a window of odd
  size centred on it, shifted inward at the grid's borders so that it always
  holds exactly kt * ky * kx keys (the start along an axis of length L is
  ``clamp(p - k // 2, 0, L - k)``); no dilation, not causal;
* within the window, plain softmax attention with scale 1 / sqrt(d);
* ``lse`` is the natural log of the window's softmax denominator.

Pins live in ``tests/test_oracle_na3d.py``.
"""
from __future__ import annotations

import numpy as np

from . import bf16_to_f64

__all__ = ["window_start", "na3d_head_ref", "na3d_ref"]


def window_start(p: int, length: int, k: int) -> int:
    """First index of the size-k window around position p on an axis of the
    given length (centred, shifted inward at the ends)."""
    if k > length or k % 2 == 0:
        raise ValueError("window size must be odd and at most the axis length")
    return min(max(p - k // 2, 0), length - k)


def na3d_head_ref(q: np.ndarray, k: np.ndarray, v: np.ndarray, grid, window, rows=None):
    """One head: q, k, v ``[T*Y*X, d]`` float64 (frame-major, row-major).
    Returns ``(out [n, d], lse [n])`` for the query rows ``rows`` (all when
    None), each attending to its own window."""
    T, Y, X = grid
    kt, ky, kx = window
    d = q.shape[1]
    scale = 1.0 / np.sqrt(d)
    rows = np.arange(T * Y * X) if rows is None else np.asarray(rows)
    out = np.empty((len(rows), d))
    lse = np.empty(len(rows))
    for n, i in enumerate(rows):
        t, rem = divmod(int(i), Y * X)
        y, x = divmod(rem, X)
        t0 = window_start(t, T, kt)
        y0 = window_start(y, Y, ky)
        x0 = window_start(x, X, kx)
        idx = np.array([(tt * Y + yy) * X + xx
                        for tt in range(t0, t0 + kt)
                        for yy in range(y0, y0 + ky)
                        for xx in range(x0, x0 + kx)])
        s = (k[idx] @ q[i]) * scale
        m = s.max()
        p = np.exp(s - m)
        den = p.sum()
        out[n] = (p @ v[idx]) / den
        lse[n] = m + np.log(den)
    return out, lse


def na3d_ref(Q, K, V, grid, window, heads=None, rows=None):
    """All heads of bf16 bit arrays ``[H, T*Y*X, d]`` (uint16); returns fp64
    ``(out, lse)`` stacked over the heads requested."""
    heads = range(Q.shape[0]) if heads is None else heads
    res = [na3d_head_ref(bf16_to_f64(Q[h]), bf16_to_f64(K[h]), bf16_to_f64(V[h]), grid, window, rows)
           for h in heads]
    return np.stack([r[0] for r in res]), np.stack([r[1] for r in res])

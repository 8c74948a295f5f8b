"""fp64 CPU oracle for query-thresholded block-sparse attention with a Taylor term.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this package: only the test suite, the smoke check in ``__graft_entry__`` and
the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, header,
table or helper with the HIP library; the two meet only in the seeded input
generator (``synth``), which holds none of the method's arithmetic.

It is written to be read against the pages, not to be fast: plain numpy in
float64 on the exact bfloat16 input values, one head at a time, using only
library matmul / exp / log / sum as steps.

Sources (cited by page title and section):

* [SOL]  "Accelerating LTX-2.5 with Sol Engine" (NVlabs Sana, Sol-Engine/LTX25),
  section "Stage 2 Optimization -- Core Technology: Sol-Attn": per-row threshold
  from block proxy-score statistics (bullet "Query-dependent thresholding"),
  pooled keys compared with the threshold during the online softmax (bullet
  "On-the-fly routing"), rejected blocks approximated by a Taylor expansion
  about the row-wise mean score (bullet "Proxy-score reuse").
* [DAI]  "LTX-2.5 at 4K, in half the time" (doubleAI), section "Attention across
  two GPUs": partial answers over halves of the keys carry their running
  maximum and sum of exponentials and merge exactly; a padded key is dropped,
  not masked.

Readings where the pages are silent (each also listed in the design notes):

* pooling is the arithmetic mean over the block's valid tokens, for K and V;
* proxy score ``p_ij = (q_i . kbar_j) / sqrt(d)`` (the scaled-logit domain, so
  ``p_ij`` is exactly the mean of the block's logits by linearity);
* ``mu_i`` and ``sigma_i`` are the mean and the population standard deviation
  (ddof = 0) of ``p_i.`` over all key blocks, the ragged last block included;
* a block is selected when ``p_ij >= tau_i`` ("at or above");
* ``beta = -inf`` is dense attention (``-inf * sigma`` is never formed);
  ``beta = +inf`` selects nothing;
* the Taylor weight of a rejected block is ``n_j e^{mu_i} (1 + p_ij - mu_i)`` on
  the pooled value ``vbar_j``, added to numerator and denominator, with ``n_j``
  the block's valid token count, applied without a clamp.  It is the
  first-order expansion ``e^s ~ e^mu (1 + s - mu)`` summed over the block's
  tokens (``sum_t s_it = n_j p_ij``), with every value replaced by ``vbar_j``;
* ``lse`` is the natural log of the full denominator (exact plus Taylor mass).

Parity pins for every function live in ``tests/test_oracle_*.py``.  Agreement
with the authors' own Sol-Attn implementation is parity unpinned: the pages
print no formula for the Taylor term and no worked numeric example.
"""
from __future__ import annotations

from typing import Iterable, Optional, Sequence

import numpy as np

__all__ = [
    "bf16_to_f64",
    "block_bounds",
    "pool_ref",
    "proxy_ref",
    "row_stats_ref",
    "select_ref",
    "near_ties_ref",
    "sol_attn_head_ref",
    "dense_head_ref",
    "lse_merge_ref",
    "sol_attn_ref",
    "sol_attn_shard_ref",
    "dense_ref",
]


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bfloat16 bit patterns (uint16) as float64."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def block_bounds(nk: int, B: int) -> list:
    """Key blocks ``[jB, min(nk, (j+1)B))``; the last one may be ragged.

    A ragged block holds only real tokens: no pad key is ever added [DAI]."""
    return [(s, min(nk, s + B)) for s in range(0, nk, B)]


def pool_ref(x: np.ndarray, B: int) -> np.ndarray:
    """Mean-pooled blocks [SOL "On-the-fly routing", "Proxy-score reuse"].

    ``x`` is ``[nk, d]``; returns ``[nb, d]`` with row ``j`` the mean of the
    block's valid tokens."""
    return np.stack([x[s:e].mean(axis=0) for s, e in block_bounds(x.shape[0], B)])


def proxy_ref(q: np.ndarray, kbar: np.ndarray) -> np.ndarray:
    """Block proxy scores ``p_ij = q_i . kbar_j / sqrt(d)`` (``[nq, nb]``) [SOL]."""
    return (q @ kbar.T) / np.sqrt(q.shape[1])


def row_stats_ref(p: np.ndarray):
    """Per-row mean and population standard deviation of the proxy scores [SOL
    "Query-dependent thresholding"]."""
    mu = p.mean(axis=1)
    sigma = np.sqrt(((p - mu[:, None]) ** 2).mean(axis=1))
    return mu, sigma


def select_ref(p: np.ndarray, mu: np.ndarray, sigma: np.ndarray, beta: float,
               force: Optional[dict] = None) -> np.ndarray:
    """Selected blocks ``p_ij >= tau_i``, ``tau_i = mu_i + beta sigma_i`` [SOL].

    ``beta = -inf`` selects every block (dense); ``beta = +inf`` selects none.
    ``force`` maps ``(row, block) -> bool`` to fix the decision on chosen pairs
    (used only to enumerate the equally valid decisions on near-ties)."""
    if np.isneginf(beta):
        sel = np.ones(p.shape, dtype=bool)
    elif np.isposinf(beta):
        sel = np.zeros(p.shape, dtype=bool)
    else:
        tau = mu + beta * sigma
        sel = p >= tau[:, None]
    if force:
        sel = sel.copy()
        for (i, j), val in force.items():
            sel[i, j] = bool(val)
    return sel


def near_ties_ref(p: np.ndarray, mu: np.ndarray, sigma: np.ndarray, beta: float,
                  eps: float) -> list:
    """Pairs ``(row, block)`` whose proxy is within ``eps`` of the threshold.

    On these pairs either decision is correct (finite-precision tie)."""
    if not np.isfinite(beta):
        return []
    tau = mu + beta * sigma
    i, j = np.nonzero(np.abs(p - tau[:, None]) < eps)
    return list(zip(i.tolist(), j.tolist()))


def sol_attn_head_ref(q: np.ndarray, k: np.ndarray, v: np.ndarray, B: int,
                      beta: float, rows: Optional[Sequence[int]] = None,
                      force: Optional[dict] = None, taylor: bool = True,
                      chunk: int = 256, pooled=None,
                      blocks: Optional[Sequence[int]] = None):
    """One head of Sol-Attn-style sparse attention, step by step [SOL].

    ``q`` ``[nq, d]``, ``k``/``v`` ``[nk, d]`` (float64).  ``rows`` restricts
    the computation to some query rows (rows are independent).  ``force`` keys
    are absolute row indices.  ``taylor=False`` drops the Taylor term (hard
    selection), for quality comparisons only.  ``pooled`` may pass the
    ``(kbar, vbar)`` this function returned in ``info`` for the same keys, to
    skip recomputing them.

    ``blocks`` restricts the exact and the Taylor sums to those key blocks --
    one rank's share of keys split along the sequence [DAI "Attention across
    two GPUs": each GPU attends to its part of the keys and the partial
    answers merge] -- while the proxy statistics ``mu``, ``sigma`` still run
    over every block of ``k`` (the thresholds of the whole sequence [SOL]).
    The result is then that share's partial answer: ``out`` = its numerator
    over its denominator, ``lse`` = reference + log of its denominator.

    Returns ``(out [R, d], lse [R], info)`` where ``info`` holds ``p``, ``mu``,
    ``sigma``, the selection ``mask`` of the computed rows and ``partial`` =
    ``(num [R, d], den [R], M [R])`` (``num``, ``den`` relative to ``e^M``).
    A row whose denominator is not positive gets NaN output (none occur on the
    workloads; a share of rejected blocks alone can have one).
    """
    nq, d = q.shape
    nk = k.shape[0]
    scale = 1.0 / np.sqrt(d)
    rows = np.arange(nq) if rows is None else np.asarray(rows, dtype=np.int64)
    bounds = block_bounds(nk, B)
    n_j = np.array([e - s for s, e in bounds], dtype=np.float64)
    # step 1: pooled keys and values
    if pooled is None:
        kbar = pool_ref(k, B)
        vbar = pool_ref(v, B)
    else:
        kbar, vbar = pooled
    # step 2: proxy scores for the requested rows
    qr = q[rows]
    p = proxy_ref(qr, kbar)
    # step 3: row statistics
    mu, sigma = row_stats_ref(p)
    # step 4: selection (forced decisions refer to absolute rows)
    local_force = None
    if force:
        pos = {int(r): i for i, r in enumerate(rows.tolist())}
        local_force = {(pos[r], j): val for (r, j), val in force.items() if r in pos}
    sel = select_ref(p, mu, sigma, beta, local_force)
    tok_block = np.repeat(np.arange(len(bounds)), n_j.astype(np.int64))
    # blocks whose keys this computation sums over (all, or one share)
    in_share = np.ones(len(bounds), dtype=bool)
    if blocks is not None:
        in_share[:] = False
        in_share[np.asarray(blocks, dtype=np.int64)] = True
    sel_in = sel & in_share[None, :]
    rej_in = ~sel & in_share[None, :]
    pnum = np.empty((len(rows), d))
    pden = np.empty(len(rows))
    pM = np.empty(len(rows))

    out = np.empty((len(rows), d))
    lse = np.empty(len(rows))
    for r0 in range(0, len(rows), chunk):
        r1 = min(len(rows), r0 + chunk)
        # step 5: exact logits
        s = scale * (qr[r0:r1] @ k.T)                      # [R, nk]
        tok_sel = sel_in[r0:r1][:, tok_block]               # [R, nk]
        # step 6: reference shift (any finite shift is exact; this one avoids overflow)
        s_sel = np.where(tok_sel, s, -np.inf)
        M = s_sel.max(axis=1)
        any_rej = rej_in[r0:r1].any(axis=1)
        M = np.where(any_rej & taylor, np.maximum(M, mu[r0:r1]), M)
        # step 7: exact part over selected blocks ...
        with np.errstate(invalid="ignore", over="ignore"):
            e = np.where(tok_sel, np.exp(s - M[:, None]), 0.0)
        num = e @ v
        den = e.sum(axis=1)
        # ... plus the first-order Taylor part over rejected blocks
        if taylor:
            dmu = p[r0:r1] - mu[r0:r1, None]
            w = n_j[None, :] * np.exp(mu[r0:r1] - M)[:, None] * (1.0 + dmu)
            w = np.where(rej_in[r0:r1], w, 0.0)
            num = num + w @ vbar
            den = den + w.sum(axis=1)
        pnum[r0:r1], pden[r0:r1], pM[r0:r1] = num, den, M
        # step 8: normalise
        ok = den > 0
        with np.errstate(invalid="ignore", divide="ignore"):
            out[r0:r1] = np.where(ok[:, None], num / den[:, None], np.nan)
            lse[r0:r1] = np.where(ok, M + np.log(np.where(ok, den, 1.0)), np.nan)
    info = dict(p=p, mu=mu, sigma=sigma, mask=sel, rows=rows, pooled=(kbar, vbar),
                partial=(pnum, pden, pM))
    return out, lse, info


def dense_head_ref(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                   rows: Optional[Sequence[int]] = None, chunk: int = 256):
    """Textbook softmax attention with scale ``1/sqrt(d)`` and its log-sum-exp."""
    nq, d = q.shape
    rows = np.arange(nq) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((len(rows), d))
    lse = np.empty(len(rows))
    for r0 in range(0, len(rows), chunk):
        r1 = min(len(rows), r0 + chunk)
        s = (q[rows[r0:r1]] @ k.T) / np.sqrt(d)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        den = e.sum(axis=1)
        out[r0:r1] = (e @ v) / den[:, None]
        lse[r0:r1] = m[:, 0] + np.log(den)
    return out, lse


def lse_merge_ref(out_a, lse_a, out_b, lse_b):
    """Exact merge of two partial answers over disjoint key sets [DAI].

    ``lse = log(e^{lse_a} + e^{lse_b})``; each output is weighted by its share
    of the total mass.  Two empty partials (both ``-inf``) give zero output
    and ``-inf``."""
    lse_a = np.asarray(lse_a, dtype=np.float64)
    lse_b = np.asarray(lse_b, dtype=np.float64)
    lse = np.logaddexp(lse_a, lse_b)
    both_empty = np.isneginf(lse)
    safe = np.where(both_empty, 0.0, lse)
    wa = np.where(both_empty, 0.0, np.exp(lse_a - safe))
    wb = np.where(both_empty, 0.0, np.exp(lse_b - safe))
    out = wa[..., None] * out_a + wb[..., None] * out_b
    return out, lse


def _heads(x: np.ndarray) -> Iterable:
    return (x[h] for h in range(x.shape[0]))


def sol_attn_ref(Q, K, V, B: int, beta: float, rows=None, taylor: bool = True):
    """All heads: ``Q`` ``[H, nq, d]``, ``K``/``V`` ``[H, nk, d]`` (bf16 bits or float)."""
    Q = Q if Q.dtype != np.uint16 else bf16_to_f64(Q)
    K = K if K.dtype != np.uint16 else bf16_to_f64(K)
    V = V if V.dtype != np.uint16 else bf16_to_f64(V)
    outs, lses = [], []
    for q, k, v in zip(_heads(Q), _heads(K), _heads(V)):
        o, l, _ = sol_attn_head_ref(q, k, v, B, beta, rows=rows, taylor=taylor)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)


def sol_attn_shard_ref(Q, K, V, B: int, beta: float, blocks: Sequence[int], rows=None):
    """All heads of one share's partial answer (``blocks`` of the key sequence,
    statistics over all blocks); ``(out, lse)`` stacked over heads."""
    Q = Q if Q.dtype != np.uint16 else bf16_to_f64(Q)
    K = K if K.dtype != np.uint16 else bf16_to_f64(K)
    V = V if V.dtype != np.uint16 else bf16_to_f64(V)
    outs, lses = [], []
    for q, k, v in zip(_heads(Q), _heads(K), _heads(V)):
        o, l, _ = sol_attn_head_ref(q, k, v, B, beta, rows=rows, blocks=blocks)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)


def dense_ref(Q, K, V, rows=None):
    """All heads of dense attention (bf16 bits or float inputs)."""
    Q = Q if Q.dtype != np.uint16 else bf16_to_f64(Q)
    K = K if K.dtype != np.uint16 else bf16_to_f64(K)
    V = V if V.dtype != np.uint16 else bf16_to_f64(V)
    outs, lses = [], []
    for q, k, v in zip(_heads(Q), _heads(K), _heads(V)):
        o, l = dense_head_ref(q, k, v, rows=rows)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)

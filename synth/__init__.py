"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

This module holds no step of the attention method: it only draws random
tensors and rounds them to bfloat16.  Both the HIP path and the CPU oracle
receive the same bytes from here.

Workload shapes stand in for LTX-2.5 latent sequences (Sol-Engine LTX25 page,
"Stage 2 Optimization -- Core Technology: Sol-Attn": video tokens with audio
tokens in the same attention; doubleAI page, "Attention across two GPUs": about
a hundred audio queries against the video keys).  The pages publish no dataset,
so every input is drawn from the recipe below.

Clustered self-attention recipe, per head ``h`` with its own generator
``default_rng(SeedSequence([seed, h]))`` (so any head can be regenerated alone),
drawn in this order, in float32:

1. ``C`` centres ``c_0..c_{C-1}`` ~ N(0, I_d);
2. key token ``t``:   ``k_t = c_{(t // B) mod C} + noise * N(0, I_d)``;
3. one centre index ``u_b`` ~ U{0..C-1} per query block ``b`` of ``B`` rows;
4. query token ``t``: ``q_t = c_{u_{t // B}} + noise * N(0, I_d)``;
5. ``v_t`` ~ N(0, I_d).

Per-token stress variant (``per_token=True``): step 3 draws one centre index
per query token instead of per query block, so neighbouring rows share no
centre and almost every query tile needs almost every key block.

Cross-attention recipe (short audio query against long video keys): per head,
Q, K, V ~ N(0, 1) drawn in that order.

All tensors are rounded to bfloat16 with round-to-nearest-even and laid out
``[H, N, d]`` contiguous.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Optional

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "clustered_head",
    "clustered",
    "cross_head",
    "cross",
    "gaussian",
]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # finite inputs: u + 0x7FFF + lsb stays below 2^32
    out = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
           >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bits to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass(frozen=True)
class Workload:
    """One attention shape. ``n_video`` tokens of clustered keys, then ``n_audio``."""

    name: str
    heads: int
    n_video: int
    n_audio: int
    head_dim: int
    block: int
    centres: int
    noise: float
    seed: int
    betas: tuple

    @property
    def n(self) -> int:
        return self.n_video + self.n_audio


# Shapes of the LTX-2.5 latent sequences: 16 latent frames of
# (24x16 | 48x32 | 120x68) patches, plus 126 audio tokens at Stage 2.
WORKLOADS = {
    "tiny": Workload("tiny", 2, 2048, 0, 128, 64, 32, 0.5, 0, (0.0, float("-inf"))),
    "stage1": Workload("stage1", 32, 6144, 0, 128, 128, 48, 0.5, 1,
                       (float("-inf"), 0.0, 0.5)),
    "stage2": Workload("stage2", 32, 24576, 126, 128, 128, 192, 0.5, 3, (0.5,)),
    "4k": Workload("4k", 32, 130560, 126, 128, 128, 1020, 0.5, 4, (0.5, 1.0)),
}

# Audio -> video cross-attention: 126 audio queries, 130,560 video keys,
# computed whole and as two halves of 65,280 keys.
CROSS = dict(heads=32, nq=126, nk=130560, head_dim=128, seed=2, split=65280)


def _head_rng(seed: int, h: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, h]))


def clustered_head(n: int, d: int, block: int, centres: int, noise: float,
                   seed: int, h: int, per_token: bool = False):
    """bf16 bits of (q, k, v), each ``[n, d]``, for head ``h`` of the clustered recipe
    (``per_token``: the stress variant with one query centre per token)."""
    rng = _head_rng(seed, h)
    c = rng.standard_normal((centres, d), dtype=np.float32)
    t = np.arange(n)
    kc = (t // block) % centres
    k = c[kc] + np.float32(noise) * rng.standard_normal((n, d), dtype=np.float32)
    if per_token:
        qc = rng.integers(0, centres, size=n)
    else:
        nqb = (n + block - 1) // block
        qc = rng.integers(0, centres, size=nqb)[t // block]
    q = c[qc] + np.float32(noise) * rng.standard_normal((n, d), dtype=np.float32)
    v = rng.standard_normal((n, d), dtype=np.float32)
    return f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)


def clustered(w: Workload, heads: Optional[list] = None, threads: int = 8,
              per_token: bool = False):
    """bf16 bits of (Q, K, V) ``[H, N, d]`` for a named workload (all heads by default).

    Heads are independent streams, so they are drawn on a thread pool."""
    hs = list(range(w.heads)) if heads is None else list(heads)
    n, d = w.n, w.head_dim
    Q = np.empty((len(hs), n, d), np.uint16)
    K = np.empty_like(Q)
    V = np.empty_like(Q)

    def one(i):
        Q[i], K[i], V[i] = clustered_head(n, d, w.block, w.centres, w.noise, w.seed, hs[i],
                                          per_token)

    if threads > 1 and len(hs) > 1:
        with ThreadPoolExecutor(min(threads, len(hs))) as ex:
            list(ex.map(one, range(len(hs))))
    else:
        for i in range(len(hs)):
            one(i)
    return Q, K, V


def cross_head(nq: int, nk: int, d: int, seed: int, h: int):
    """bf16 bits of (q ``[nq,d]``, k ``[nk,d]``, v ``[nk,d]``) for one head, N(0,1)."""
    rng = _head_rng(seed, h)
    q = rng.standard_normal((nq, d), dtype=np.float32)
    k = rng.standard_normal((nk, d), dtype=np.float32)
    v = rng.standard_normal((nk, d), dtype=np.float32)
    return f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)


def cross(heads: int, nq: int, nk: int, d: int, seed: int, threads: int = 8):
    Q = np.empty((heads, nq, d), np.uint16)
    K = np.empty((heads, nk, d), np.uint16)
    V = np.empty((heads, nk, d), np.uint16)

    def one(h):
        Q[h], K[h], V[h] = cross_head(nq, nk, d, seed, h)

    with ThreadPoolExecutor(max(1, min(threads, heads))) as ex:
        list(ex.map(one, range(heads)))
    return Q, K, V


def gaussian(heads: int, n: int, d: int, seed: int, nk: Optional[int] = None,
             scale: float = 1.0):
    """Unclustered bf16 N(0, scale^2) inputs (Q ``[H,n,d]``, K/V ``[H,nk,d]``)."""
    nk = n if nk is None else nk
    Q = np.empty((heads, n, d), np.uint16)
    K = np.empty((heads, nk, d), np.uint16)
    V = np.empty((heads, nk, d), np.uint16)
    for h in range(heads):
        rng = _head_rng(seed, h)
        Q[h] = f32_to_bf16_bits(np.float32(scale) * rng.standard_normal((n, d), dtype=np.float32))
        K[h] = f32_to_bf16_bits(np.float32(scale) * rng.standard_normal((nk, d), dtype=np.float32))
        V[h] = f32_to_bf16_bits(rng.standard_normal((nk, d), dtype=np.float32))
    return Q, K, V


def activations(m: int, k: int, seed: int) -> np.ndarray:
    """bf16 bits ``[m, k]`` of projection inputs: N(0, 1) rows, each row scaled
    by its own power of two in [2^-6, 2^6], and a few channels 8x larger than
    the rest (the outlier channels of transformer activations)."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 0xF8]))
    x = rng.standard_normal((m, k), dtype=np.float32)
    x *= np.exp2(rng.integers(-6, 7, (m, 1))).astype(np.float32)
    x[:, rng.choice(k, size=max(1, k // 256), replace=False)] *= np.float32(8)
    return f32_to_bf16_bits(x)


def e4m3_codes(m: int, k: int, seed: int) -> np.ndarray:
    """Uniformly random E4M3 byte codes ``[m, k]``, the two NaN patterns
    (0x7F, 0xFF) excluded."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 0xE4]))
    c = rng.integers(0, 254, (m, k), dtype=np.uint16)
    c = c + (c >= 0x7F) + (c >= 0xFE)  # skip 0x7F and 0xFF
    return c.astype(np.uint8)

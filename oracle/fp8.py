"""fp64 CPU oracle for the FP8 projection GEMM with per-row activation scales.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this module: only the test suite and the ``cpu_baseline`` leg of ``bench.py``
use it.  It shares no code, header, table or helper with the HIP library.

Source: [DAI] "LTX-2.5 at 4K, in half the time" (doubleAI), section "Thinner
seams", the paragraph on the refinement pass's matrix multiplies: the weights
stay in FP8, the activations are converted to FP8 with one scale per row, and
the products accumulate in FP32, so the matrix units run at their FP8 rate.

Readings where the page is silent (each also listed in the design notes):

* the FP8 format is E4M3 in its finite-only form (bias 7, 3 mantissa bits,
  subnormals, largest finite value 448, no infinities, S.1111.111 is NaN);
* a row's scale is ``s = amax / 448`` and its codes are
  ``RNE_e4m3(x * (448 / amax))``: the row maximum maps onto the largest finite
  value.  Both quotients and the product are formed in float32 (the precision
  the activations arrive in after the bf16 -> fp32 widening), so the code of
  every element is decided in float32 on both sides; an all-zero row gets
  scale 0 and all-zero codes;
* the weights carry one scale per output channel (``sw``), quantised by the
  same rule along their input dimension;
* ``y[i, n] = sa[i] * sw[n] * sum_k dec(a[i, k]) * dec(w[n, k])``, rounded once
  to bf16 (round to nearest even).  No bias term.

The sum of E4M3 products is exact in float64 (every product has at most 8
significant bits between 2^-18 and 2^18; 2^12 of them span fewer than 53
bits), so ``fp8_gemm_ref`` returns the exact value before the final scaling.

Pins for every function live in ``tests/test_oracle_fp8.py``.
"""
from __future__ import annotations

import numpy as np

from . import bf16_to_f64

__all__ = [
    "E4M3_MAX",
    "e4m3_decode",
    "e4m3_encode",
    "quantize_rows_ref",
    "fp8_gemm_ref",
]

E4M3_MAX = 448.0


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Value of each E4M3 code (float64); NaN for S.1111.111."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = (1.0 + m / 8.0) * np.exp2(e - 7.0)
    sub = (m / 8.0) * 2.0 ** -6
    val = np.where(e == 0, sub, normal)
    val = np.where((e == 0xF) & (m == 0x7), np.nan, val)
    return sign * val


# The 127 non-negative finite values with their codes, ascending.
_POS_CODES = np.arange(0x7F, dtype=np.uint8)
_POS_VALUES = e4m3_decode(_POS_CODES)


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Round each value to the nearest E4M3 value, ties to the even code (the
    one whose mantissa ends in 0).  |x| must stay below 464, the midpoint
    between 448 and the next step of the exponent: values in (448, 464) round
    to 448, as a row's scaled maximum may land a float32 ulp above 448."""
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any() or (np.abs(x) >= 464.0).any():
        raise ValueError("e4m3_encode: input outside (-464, 464)")
    a = np.abs(x)
    hi = np.clip(np.searchsorted(_POS_VALUES, a, side="left"), 0, len(_POS_VALUES) - 1)
    lo = np.clip(hi - 1, 0, None)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((_POS_CODES[hi] & 1) == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    return np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)


def quantize_rows_ref(x_bits: np.ndarray):
    """Per-row FP8 quantisation of a bf16 matrix ``[M, K]`` (given as uint16
    bit patterns).  Returns ``(codes [M, K] uint8, scale [M] float32)``."""
    x = bf16_to_f64(x_bits).astype(np.float32)  # exact: every bf16 value is an fp32 value
    amax = np.abs(x).max(axis=1).astype(np.float32)
    safe = np.where(amax > 0, amax, np.float32(1))
    inv = np.where(amax > 0, np.float32(E4M3_MAX) / safe, np.float32(0)).astype(np.float32)
    scaled = (x * inv[:, None]).astype(np.float32)  # float32 product, as on the device
    codes = e4m3_encode(scaled.astype(np.float64))
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    return codes, scale


def fp8_gemm_ref(a_codes: np.ndarray, sa: np.ndarray, w_codes: np.ndarray, sw: np.ndarray):
    """``(y, bound)``: the exact product ``sa[i] sw[n] sum_k a[i,k] w[n,k]`` in
    float64, and a bound on what float32 accumulation of the K products in any
    order may add to it: ``K * 2^-24 * |sa| |sw| sum_k |a w|``."""
    a = e4m3_decode(a_codes)
    w = e4m3_decode(w_codes)
    acc = a @ w.T
    mag = np.abs(a) @ np.abs(w).T
    s = np.asarray(sa, dtype=np.float64)[:, None] * np.asarray(sw, dtype=np.float64)[None, :]
    k = a.shape[1]
    return s * acc, np.abs(s) * mag * (k * 2.0 ** -24)

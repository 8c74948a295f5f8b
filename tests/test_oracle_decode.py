"""Pins of the oracle's input decoding and of its multi-head entry points.

Every parity comparison starts with ``oracle.bf16_to_f64``: it turns the bf16
bit patterns the GPU receives into the fp64 values the oracle computes on.  It
is pinned here against PyTorch's own bfloat16 -> float64 conversion on all
65,536 bit patterns, and against values the bfloat16 format fixes by
definition (1 sign, 8 exponent and 7 fraction bits, bias 127).

The multi-head wrappers (``sol_attn_ref``, ``sol_attn_shard_ref``,
``dense_ref``, ``na3d.na3d_ref``) decode their bf16 inputs and stack one result
per head.  They are pinned against computations that share none of their code:
PyTorch's fp64 attention per head (a library special case), and the pure-Python
loops of the other pin files, fed with inputs decoded by PyTorch.  Each head
gets different data, so a head mix-up or a mis-decoded operand fails.

Planted mistakes (half-precision instead of bfloat16, a wrong shift, byte
order swapped, the sign bit dropped, fraction bits truncated) must each fail
the decoder pin.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from oracle import na3d as NA
from synth import f32_to_bf16_bits
from tests.test_oracle_na3d import _brute as brute_na3d
from tests.test_oracle_pins import brute_sparse
from tests.test_oracle_shard import _brute_share

ALL_BITS = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def _torch_decode(bits):
    """PyTorch's bfloat16 -> float64 conversion of uint16 bit patterns."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def _decoder_matches_torch(decode):
    got = np.asarray(decode(ALL_BITS), dtype=np.float64)
    ref = _torch_decode(ALL_BITS)
    if got.shape != ref.shape:
        return False
    nan_ok = np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    return bool(nan_ok and np.array_equal(got[fin], ref[fin])
                and np.array_equal(np.signbit(got[fin]), np.signbit(ref[fin])))


def test_bf16_decode_all_patterns_match_torch():
    """All 65,536 patterns: equal values (signed zeros, infinities and
    subnormals included), NaN at exactly the same positions."""
    assert _decoder_matches_torch(O.bf16_to_f64)
    # 2 x 127 NaN payloads per sign: exponent all ones, fraction non-zero
    assert int(np.isnan(O.bf16_to_f64(ALL_BITS)).sum()) == 2 * 127


@pytest.mark.parametrize("bits,value", [
    (0x3F80, 1.0),
    (0xC000, -2.0),
    (0x3F81, 1.0 + 2.0 ** -7),                 # one fraction ulp above 1
    (0x7F7F, (2.0 - 2.0 ** -7) * 2.0 ** 127),  # largest finite
    (0x0080, 2.0 ** -126),                     # smallest normal
    (0x0001, 2.0 ** -133),                     # smallest subnormal
    (0x807F, -(2.0 ** -126 - 2.0 ** -133)),    # largest negative subnormal
    (0x7F80, math.inf),
    (0xFF80, -math.inf),
])
def test_bf16_decode_format_values(bits, value):
    """Values fixed by the format: (-1)^s 2^(e-127) (1 + f/128), subnormals
    2^-126 (f/128)."""
    got = O.bf16_to_f64(np.array([bits], dtype=np.uint16))[0]
    assert got == value


def test_bf16_decode_signed_zero():
    z = O.bf16_to_f64(np.array([0x0000, 0x8000], dtype=np.uint16))
    assert z[0] == 0.0 and z[1] == 0.0
    assert not np.signbit(z[0]) and np.signbit(z[1])


def test_bf16_decode_round_trips_the_generator():
    """Decoding the generator's bf16 rounding of fp32 values returns torch's
    bf16 rounding of the same values."""
    x = np.random.default_rng(3).standard_normal(4096).astype(np.float32) * 7
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.bf16_to_f64(f32_to_bf16_bits(x)), ref)


def _mutant_decoder(kind):
    def dec(bits):
        b = np.asarray(bits, dtype=np.uint16)
        if kind == "as_half":
            return b.view(np.float16).astype(np.float64)
        if kind == "shift_15":
            return (b.astype(np.uint32) << np.uint32(15)).view(np.float32).astype(np.float64)
        if kind == "byte_swap":
            b = b.byteswap()
        elif kind == "no_sign":
            b = b & np.uint16(0x7FFF)
        elif kind == "truncated_fraction":
            b = b & np.uint16(0xFFF0)
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return dec


@pytest.mark.parametrize("kind", ["as_half", "shift_15", "byte_swap", "no_sign",
                                  "truncated_fraction"])
def test_planted_decoder_mistakes_are_caught(kind):
    assert not _decoder_matches_torch(_mutant_decoder(kind))


def test_unmutated_decoder_copy_passes():
    assert _decoder_matches_torch(_mutant_decoder("none"))


# --------------------------------------------------------------------------
# multi-head entry points
# --------------------------------------------------------------------------


def _bf16_heads(seed, H, n, d, scale=1.0):
    x = np.random.default_rng(seed).standard_normal((H, n, d)).astype(np.float32) * scale
    return f32_to_bf16_bits(x)


def _torch_attention(qb, kb, vb):
    """fp64 attention of one head from PyTorch (inputs decoded by PyTorch)."""
    q, k, v = (torch.from_numpy(_torch_decode(x)) for x in (qb, kb, vb))
    out = torch.nn.functional.scaled_dot_product_attention(q[None], k[None], v[None])[0]
    lse = torch.logsumexp(q @ k.T / math.sqrt(q.shape[1]), dim=1)
    return out.numpy(), lse.numpy()


def test_dense_ref_heads_match_torch_attention():
    Q, K, V = (_bf16_heads(s, 3, n, 32) for s, n in ((1, 20), (2, 45), (3, 45)))
    out, lse = O.dense_ref(Q, K, V)
    assert out.shape == (3, 20, 32) and lse.shape == (3, 20)
    for h in range(3):
        o, l = _torch_attention(Q[h], K[h], V[h])
        np.testing.assert_allclose(out[h], o, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[h], l, rtol=0, atol=1e-12)
    rows = [0, 7, 19]
    ro, rl = O.dense_ref(Q, K, V, rows=rows)
    np.testing.assert_array_equal(ro, out[:, rows])
    np.testing.assert_array_equal(rl, lse[:, rows])


def test_sol_attn_ref_dense_limit_heads_match_torch_attention():
    Q, K, V = (_bf16_heads(s, 3, n, 32) for s, n in ((4, 16), (5, 50), (6, 50)))
    out, lse = O.sol_attn_ref(Q, K, V, 8, -math.inf)
    for h in range(3):
        o, l = _torch_attention(Q[h], K[h], V[h])
        np.testing.assert_allclose(out[h], o, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[h], l, rtol=0, atol=1e-12)


@pytest.mark.parametrize("beta", [0.0, 0.5])
def test_sol_attn_ref_heads_match_bruteforce(beta):
    """Tiny 3-head sparse call (ragged last block) against the pure-Python loops
    of the method, one head at a time, on PyTorch-decoded inputs."""
    B, d = 4, 8
    Q, K, V = (_bf16_heads(s, 3, n, d, 2.0) for s, n in ((7, 6), (8, 18), (9, 18)))
    out, lse = O.sol_attn_ref(Q, K, V, B, beta)
    for h in range(3):
        q, k, v = (_torch_decode(x[h]).tolist() for x in (Q, K, V))
        bo, bl, _ = brute_sparse(q, k, v, B, beta)
        np.testing.assert_allclose(out[h], bo, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(lse[h], bl, rtol=1e-10, atol=1e-12)


def test_sol_attn_shard_ref_heads_match_bruteforce():
    B, d, beta = 4, 8, 0.5
    Q, K, V = (_bf16_heads(s, 3, n, d, 2.0) for s, n in ((10, 5), (11, 22), (12, 22)))
    share = [1, 3, 5]  # blocks of the 6 (the last one ragged: 2 keys)
    out, lse = O.sol_attn_shard_ref(Q, K, V, B, beta, blocks=share)
    for h in range(3):
        q, k, v = (_torch_decode(x[h]).tolist() for x in (Q, K, V))
        bo, bl = _brute_share(q, k, v, B, beta, share)
        np.testing.assert_allclose(out[h], bo, rtol=1e-10, atol=1e-12, equal_nan=True)
        np.testing.assert_allclose(lse[h], bl, rtol=1e-10, atol=1e-12, equal_nan=True)


def test_na3d_ref_heads_match_bruteforce():
    grid, window, d = (3, 4, 5), (3, 3, 3), 8
    n = int(np.prod(grid))
    Q, K, V = (_bf16_heads(s, 3, n, d) for s in (13, 14, 15))
    out, lse = NA.na3d_ref(Q, K, V, grid, window)
    for h in range(3):
        q, k, v = (_torch_decode(x[h]) for x in (Q, K, V))
        bo, bl = brute_na3d(q, k, v, grid, window)
        np.testing.assert_allclose(out[h], bo, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse[h], bl, rtol=1e-12, atol=1e-12)
    part, lp = NA.na3d_ref(Q, K, V, grid, window, heads=[2, 0], rows=[0, 31, n - 1])
    np.testing.assert_array_equal(part, out[[2, 0]][:, [0, 31, n - 1]])
    np.testing.assert_array_equal(lp, lse[[2, 0]][:, [0, 31, n - 1]])

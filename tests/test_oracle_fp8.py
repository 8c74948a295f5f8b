"""Pins of the FP8 GEMM oracle (``oracle.fp8``) against what the E4M3 format
definition, an independent library conversion and exact integer arithmetic
fix.  CPU only."""
import numpy as np
import pytest

import oracle.fp8 as F

torch = pytest.importorskip("torch")


def test_decode_fixed_points_of_the_format():
    # sign, 4 exponent bits (bias 7), 3 mantissa bits; subnormals at exponent 0
    cases = {0x00: 0.0, 0x38: 1.0, 0xB8: -1.0, 0x7E: 448.0, 0xFE: -448.0,
             0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x3C: 1.5,
             0x40: 2.0, 0x44: 3.0, 0x30: 0.5, 0x77: 240.0}
    for c, v in cases.items():
        assert F.e4m3_decode(np.array([c], np.uint8))[0] == v, hex(c)
    assert np.isnan(F.e4m3_decode(np.array([0x7F, 0xFF], np.uint8))).all()
    vals = F.e4m3_decode(np.arange(256, dtype=np.uint8))
    assert np.isfinite(vals).sum() == 254
    pos = vals[:0x7F]
    assert (np.diff(pos) > 0).all()  # codes 0..126 ascend strictly


def test_encode_matches_torch_float8_e4m3fn():
    """Round to nearest even against torch's own float8 conversion, on random
    values and on every midpoint between neighbouring representable values."""
    rng = np.random.default_rng(11)
    x = np.concatenate([
        rng.uniform(-448, 448, 50000),
        rng.standard_normal(50000) * 2.0 ** rng.integers(-12, 8, 50000),
    ]).astype(np.float32)
    pos = F.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids, pos.astype(np.float32), [0.0, -0.0]]).astype(np.float32)
    x = np.clip(x, -448, 448)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = F.e4m3_encode(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_encode_decode_round_trip_and_range():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    assert np.array_equal(F.e4m3_encode(F.e4m3_decode(codes)), codes)
    # a scaled row maximum may land just above 448: it rounds to 448
    assert F.e4m3_encode(np.array([448.00003, -463.9]))[0] == 0x7E
    assert F.e4m3_encode(np.array([-463.9]))[0] == 0xFE
    with pytest.raises(ValueError):
        F.e4m3_encode(np.array([464.0]))


def _bf16_bits(x):
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_quantize_rows_maps_row_max_to_448_and_bounds_the_error():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((40, 256)).astype(np.float32) * 2.0 ** rng.integers(-20, 20, (40, 1))
    x[5] = 0.0                      # all-zero row
    x[6] = 0.0
    x[6, 17] = -3.0                 # one non-zero element
    bits = _bf16_bits(x)
    xf = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    codes, scale = F.quantize_rows_ref(bits)
    assert scale.dtype == np.float32
    assert scale[5] == 0 and not codes[5].any()
    assert codes[6, 17] == 0xFE and (np.delete(codes[6], 17) == 0).all()
    for i in range(40):
        if i == 5:
            continue
        j = np.argmax(np.abs(xf[i]))
        assert F.e4m3_decode(codes[i, j:j + 1])[0] == np.copysign(448.0, xf[i, j])
        deq = scale[i] * F.e4m3_decode(codes[i])
        # half an ulp of a 3-bit mantissa (relative 2^-4) in the normal range,
        # half the subnormal spacing 2^-10 below it, plus the float32 scalings
        tol = np.maximum(np.abs(xf[i]) * 2.0 ** -4, scale[i] * 2.0 ** -10) * (1 + 1e-6)
        assert (np.abs(deq - xf[i]) <= tol).all()


def test_gemm_equals_exact_integer_dot_products():
    """Every E4M3 value is an integer multiple of 2^-9, so the dot products are
    exact in Python integers: the oracle must agree bit for bit."""
    rng = np.random.default_rng(5)
    M, N, K = 5, 7, 64
    a = rng.integers(0, 256, (M, K)).astype(np.uint8)
    w = rng.integers(0, 256, (N, K)).astype(np.uint8)
    a[(a & 0x7F) == 0x7F] = 0x12    # no NaN codes
    w[(w & 0x7F) == 0x7F] = 0x34
    sa = rng.uniform(0.5, 2, M).astype(np.float32)
    sw = rng.uniform(0.5, 2, N).astype(np.float32)
    y, bound = F.fp8_gemm_ref(a, sa, w, sw)
    ia = (F.e4m3_decode(a) * 2 ** 9).astype(np.int64)
    iw = (F.e4m3_decode(w) * 2 ** 9).astype(np.int64)
    for i in range(M):
        for n in range(N):
            exact = sum(int(ia[i, k]) * int(iw[n, k]) for k in range(K))
            assert y[i, n] == float(sa[i]) * float(sw[n]) * (exact / 2.0 ** 18)
    assert (bound >= 0).all()


def test_gemm_with_identity_weights_returns_the_dequantised_rows():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((6, 128)).astype(np.float32)
    codes, sa = F.quantize_rows_ref(_bf16_bits(x))
    w = np.zeros((128, 128), np.uint8)
    np.fill_diagonal(w, 0x38)  # 1.0
    y, _ = F.fp8_gemm_ref(codes, sa, w, np.ones(128, np.float32))
    assert np.array_equal(y, sa[:, None].astype(np.float64) * F.e4m3_decode(codes))

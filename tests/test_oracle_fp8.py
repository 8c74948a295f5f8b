"""Pins of the FP8 GEMM oracle (``oracle.fp8``) against what the E4M3 format
definition, an independent library conversion and exact integer arithmetic
fix.  CPU only.

Each pin is a checker taking the oracle module, so that the same checks also
run on mutated copies of the oracle (a wrong exponent bias or subnormal step,
ties rounded the wrong way, a signed row maximum, an inverted or dropped scale,
untransposed weights): ``test_planted_mistakes_are_caught`` requires every
mutant to fail at least one of them."""
import os
import types

import numpy as np
import pytest

import oracle.fp8 as F0

torch = pytest.importorskip("torch")


def _decode_fixed_points(F):
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


def _encode_matches_torch(F):
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


def _round_trip_and_range(F):
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    assert np.array_equal(F.e4m3_encode(F.e4m3_decode(codes)), codes)
    # a scaled row maximum may land just above 448: it rounds to 448
    assert F.e4m3_encode(np.array([448.00003, -463.9]))[0] == 0x7E
    assert F.e4m3_encode(np.array([-463.9]))[0] == 0xFE
    with pytest.raises(ValueError):
        F.e4m3_encode(np.array([464.0]))


def _bf16_bits(x):
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _quantize_rows(F):
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


def _gemm_exact_integers(F):
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


def _gemm_identity(F):
    rng = np.random.default_rng(9)
    x = rng.standard_normal((6, 128)).astype(np.float32)
    codes, sa = F.quantize_rows_ref(_bf16_bits(x))
    w = np.zeros((128, 128), np.uint8)
    np.fill_diagonal(w, 0x38)  # 1.0
    y, _ = F.fp8_gemm_ref(codes, sa, w, np.ones(128, np.float32))
    assert np.array_equal(y, sa[:, None].astype(np.float64) * F.e4m3_decode(codes))


PINS = {
    "decode_fixed_points": _decode_fixed_points,
    "encode_matches_torch": _encode_matches_torch,
    "round_trip_and_range": _round_trip_and_range,
    "quantize_rows": _quantize_rows,
    "gemm_exact_integers": _gemm_exact_integers,
    "gemm_identity": _gemm_identity,
}


@pytest.mark.parametrize("name", list(PINS))
def test_pin(name):
    """Decode: fixed points of the format.  Encode: torch's float8_e4m3fn
    conversion on random values and every midpoint.  Quantisation: the row
    maximum maps to 448 and the error stays within half a code step.  GEMM:
    exact integer dot products and identity weights."""
    PINS[name](F0)


# --------------------------------------------------------------------------
# the pins above catch planted mistakes (mutated copies of the oracle, on the CPU)
# --------------------------------------------------------------------------

_MUTANTS = {
    "exponent_bias_8": ("np.exp2(e - 7.0)", "np.exp2(e - 8.0)"),
    "subnormal_scale": ("sub = (m / 8.0) * 2.0 ** -6", "sub = (m / 8.0) * 2.0 ** -7"),
    "ties_away": ("((d_hi == d_lo) & ((_POS_CODES[hi] & 1) == 0))", "(d_hi == d_lo)"),
    "ties_down": ("((d_hi == d_lo) & ((_POS_CODES[hi] & 1) == 0))", "False"),
    "signed_max": ("amax = np.abs(x).max(axis=1)", "amax = x.max(axis=1)"),
    "scale_inverted": ("scale = (amax / np.float32(E4M3_MAX))", "scale = (np.float32(E4M3_MAX) / safe)"),
    "weight_scale_dropped": ("* np.asarray(sw, dtype=np.float64)[None, :]", "* 1.0"),
    "weights_untransposed": ("acc = a @ w.T", "acc = a @ w"),
}


def _mutant_module(kind):
    old, new = _MUTANTS[kind]
    path = os.path.join(os.path.dirname(F0.__file__), "fp8.py")
    src = open(path).read()
    assert src.count(old) == 1, kind
    m = types.ModuleType(f"fp8_mutant_{kind}")
    m.__package__ = "oracle"  # the copy imports the oracle's pinned bf16 decoder
    exec(compile(src.replace(old, new), f"<fp8 mutant {kind}>", "exec"), m.__dict__)
    return m


@pytest.mark.parametrize("kind", list(_MUTANTS))
def test_planted_mistakes_are_caught(kind):
    """Each mutated copy of the FP8 oracle must fail at least one pin."""
    m = _mutant_module(kind)
    failed = []
    for name, pin in PINS.items():
        try:
            pin(m)
        except (AssertionError, ValueError, IndexError):
            failed.append(name)
    assert failed, f"planted mistake {kind!r} passed every pin"


def test_unmutated_copy_passes_every_pin():
    """The copying mechanism itself changes nothing."""
    m = types.ModuleType("fp8_copy")
    m.__package__ = "oracle"
    path = os.path.join(os.path.dirname(F0.__file__), "fp8.py")
    exec(compile(open(path).read(), "<fp8 copy>", "exec"), m.__dict__)
    for pin in PINS.values():
        pin(m)

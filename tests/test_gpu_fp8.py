"""GPU parity of the FP8 projection GEMM entry points against ``oracle.fp8``.

Quantisation: codes and scales bit-exact (the code of every element is decided
in float32 on both sides).  GEMM: each bf16 output within
``2^-8 |y| (1.001) + 2 * bound``, where ``y`` is the oracle's exact value and
``bound`` its bound on float32 accumulation of the K products in any order:
one bf16 rounding (unit roundoff 2^-8) on top of the accumulation error.
Inputs come from the seeded generator and the oracle's own quantisation, never
from the GPU.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import block_sparse_attention_06_amd as sa  # noqa: E402
import oracle.fp8 as F  # noqa: E402
from synth import activations, e4m3_codes  # noqa: E402

pytestmark = pytest.mark.gpu


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _bf16_to_f64(t):
    return (t.view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32) << 16).view(
        np.float32).astype(np.float64)


@pytest.mark.parametrize("M,K", [(1, 128), (37, 4096), (1000, 520), (5, 8), (9, 4104), (3, 8192)])
def test_quantize_rows_bit_exact(M, K):
    x = activations(M, K, seed=M + K)
    x[0, :] = 0                                   # all-zero row
    if M > 2:
        x[1, :] = 0
        x[1, K // 2] = 0xC040                     # one element, -3.0
        x[2, :] = (np.arange(K) % 2 * 0x3F80 + 0x0001).astype(np.uint16)  # tiny vs 1.0
    codes, scale = sa.fp8_quantize_rows(_dev(x.view(np.int16)).view(torch.bfloat16))
    torch.cuda.synchronize()
    rc, rs = F.quantize_rows_ref(x)
    got_c = codes.cpu().numpy()
    got_s = scale.cpu().numpy()
    assert np.array_equal(got_s.view(np.uint32), rs.view(np.uint32))
    bad = np.argwhere(got_c != rc)
    assert bad.size == 0, f"{len(bad)} code mismatches, first at {bad[:3].tolist()}"


def _gemm_case(M, N, K, seed):
    xa = activations(M, K, seed)
    xw = activations(N, K, seed + 1)
    a, s_a = F.quantize_rows_ref(xa)
    w, s_w = F.quantize_rows_ref(xw)
    y = sa.fp8_gemm_rowscale(_dev(a), _dev(s_a), _dev(w), _dev(s_w))
    torch.cuda.synchronize()
    ref, bound = F.fp8_gemm_ref(a, s_a, w, s_w)
    got = _bf16_to_f64(y)
    tol = 2.0 ** -8 * np.abs(ref) * 1.001 + 2 * bound
    err = np.abs(got - ref)
    assert (err <= tol).all(), (
        f"M{M} N{N} K{K}: {(err > tol).sum()} outputs outside the bound, worst "
        f"{(err / np.maximum(tol, 1e-30)).max():.3g}x")


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (300, 256, 512), (513, 128, 256),
                                   (777, 384, 4096), (256, 512, 1024)])
def test_gemm_parity(M, N, K):
    _gemm_case(M, N, K, seed=M * 7 + N + K)


def test_gemm_full_projection_shape_sampled():
    """The 4K projection shape (130,686 tokens, 4096 -> 4096) on random codes and
    scales; rows sampled across the token range, every column checked."""
    M, N, K = 130686, 4096, 4096
    a = e4m3_codes(M, K, seed=1)
    w = e4m3_codes(N, K, seed=2)
    rng = np.random.default_rng(3)
    s_a = np.exp2(rng.uniform(-12, -4, M)).astype(np.float32)
    s_w = np.exp2(rng.uniform(-12, -4, N)).astype(np.float32)
    y = sa.fp8_gemm_rowscale(_dev(a), _dev(s_a), _dev(w), _dev(s_w))
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, M, 4099), [M - 1, M - 2, 255, 256]]))
    ref, bound = F.fp8_gemm_ref(a[rows], s_a[rows], w, s_w)
    got = _bf16_to_f64(y[torch.from_numpy(rows).cuda()])
    tol = 2.0 ** -8 * np.abs(ref) * 1.001 + 2 * bound
    assert (np.abs(got - ref) <= tol).all()


def test_gemm_zero_scale_rows_give_zero():
    M, N, K = 64, 128, 128
    a = e4m3_codes(M, K, seed=4)
    w = e4m3_codes(N, K, seed=5)
    s_a = np.ones(M, np.float32)
    s_a[::3] = 0.0
    y = sa.fp8_gemm_rowscale(_dev(a), _dev(s_a), _dev(w), _dev(np.ones(N, np.float32)))
    torch.cuda.synchronize()
    assert (y[::3].float() == 0).all()

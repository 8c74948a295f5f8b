"""The C ABI without a GPU: the library loads, exports every declared symbol,
and rejects bad arguments with the documented codes before launching anything
(argument checks touch no HIP API, so these run on the CPU)."""
import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "solattn.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\**\s+\**([a-z_0-9]+)\s*\(",
                                 text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    import block_sparse_attention_06_amd as sa
    return sa.load_library()


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("sol_attn_pool", "sol_attn_forward", "attn_lse_merge", "sol_attn_row_stats",
              "sol_attn_row_stats_moment", "sol_attn_workspace_size", "sol_attn_error_string", "sol_attn_proxy_scores",
              "sol_attn_block_mask", "fp8_quantize_rows", "fp8_gemm_rowscale", "na3d_forward",
              "sol_attn_forward_shard", "sol_attn_shard_workspace_size",
              "sol_attn_combine_partials", "sol_attn_tile_schedule"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for n in _declared():
        assert hasattr(lib, n), f"libsolattn.so does not export {n}"


def test_error_strings(lib):
    for code in (0, -1, -2, -3, -4, 7):
        assert len(lib.sol_attn_error_string(code)) > 0


FAKE = ctypes.c_void_p(0x10000)  # aligned, never dereferenced: checks fail first


def test_forward_argument_errors(lib):
    f = lib.sol_attn_forward
    N = None
    # null pointers
    assert f(N, FAKE, FAKE, FAKE, N, 64, 1, 128, 64, 0.0, 1, 0, FAKE, 1 << 20, N) == -1
    # bad sizes
    assert f(FAKE, FAKE, FAKE, FAKE, N, 0, 1, 128, 64, 0.0, 1, 0, FAKE, 1 << 20, N) == -1
    assert f(FAKE, FAKE, FAKE, FAKE, N, 64, -1, 128, 64, 0.0, 1, 0, FAKE, 1 << 20, N) == -1
    # unsupported head dim, block, mode
    assert f(FAKE, FAKE, FAKE, FAKE, N, 64, 1, 64, 64, 0.0, 1, 0, FAKE, 1 << 20, N) == -2
    assert f(FAKE, FAKE, FAKE, FAKE, N, 64, 1, 128, 32, 0.0, 1, 0, FAKE, 1 << 20, N) == -2
    assert f(FAKE, FAKE, FAKE, FAKE, N, 64, 1, 128, 64, 0.0, 2, 0, FAKE, 1 << 20, N) == -2
    # NaN beta
    assert f(FAKE, FAKE, FAKE, FAKE, N, 64, 1, 128, 64, math.nan, 1, 0, FAKE, 1 << 20, N) == -1
    # short or missing workspace
    need = lib.sol_attn_workspace_size(64, 64, 1, 128, 64, 1)
    assert need > 0
    assert f(FAKE, FAKE, FAKE, FAKE, N, 64, 1, 128, 64, 0.0, 1, 0, FAKE, need - 1, N) == -1
    assert f(FAKE, FAKE, FAKE, FAKE, N, 64, 1, 128, 64, 0.0, 1, 0, N, need, N) == -1
    # misaligned tensor or workspace
    mis = ctypes.c_void_p(0x10002)
    assert f(mis, FAKE, FAKE, FAKE, N, 64, 1, 128, 64, 0.0, 1, 0, FAKE, need, N) == -1
    assert f(FAKE, FAKE, FAKE, FAKE, N, 64, 1, 128, 64, 0.0, 1, 0, ctypes.c_void_p(0x10010),
             need, N) == -1


def test_other_entry_points_argument_errors(lib):
    N = None
    assert lib.sol_attn_pool(N, FAKE, FAKE, FAKE, 64, 1, 128, 64, N) == -1
    assert lib.sol_attn_pool(FAKE, FAKE, FAKE, FAKE, 64, 1, 96, 64, N) == -2
    assert lib.sol_attn_pool(FAKE, FAKE, FAKE, FAKE, 64, 1, 128, 100, N) == -2
    assert lib.sol_attn_row_stats(FAKE, N, FAKE, FAKE, 64, 64, 1, 128, 64, N) == -1
    need = 2 * 128 * 128 * 2 + 128 * 4 + 8 * (128 * 128 + 2 * 128) * 4  # one head
    rsm = lib.sol_attn_row_stats_moment
    assert rsm(FAKE, FAKE, FAKE, FAKE, 64, 64, 1, 128, 64, N, need, N) == -1      # no workspace
    assert rsm(FAKE, FAKE, FAKE, FAKE, 64, 64, 1, 128, 64, FAKE, need - 1, N) == -1  # too small
    assert rsm(FAKE, FAKE, FAKE, FAKE, 64, 64, 1, 96, 64, FAKE, need, N) == -2
    na = lib.na3d_forward
    assert na(N, FAKE, FAKE, FAKE, N, 2, 8, 8, 1, 128, 1, 3, 3, N) == -1        # null q
    assert na(FAKE, FAKE, FAKE, FAKE, N, 2, 8, 8, 1, 128, 2, 3, 3, N) == -1     # even window
    assert na(FAKE, FAKE, FAKE, FAKE, N, 2, 8, 8, 1, 128, 3, 3, 3, N) == -1     # window > T
    assert na(FAKE, FAKE, FAKE, FAKE, N, 2, 8, 40, 1, 128, 1, 3, 27, N) == -2   # kx > 25
    assert na(FAKE, FAKE, FAKE, FAKE, N, 2, 8, 8, 1, 64, 1, 3, 3, N) == -2      # d != 128
    assert lib.fp8_quantize_rows(N, FAKE, FAKE, ctypes.c_int64(4), 128, N) == -1
    assert lib.fp8_quantize_rows(FAKE, FAKE, FAKE, ctypes.c_int64(4), 12, N) == -2  # K % 8
    assert lib.fp8_gemm_rowscale(FAKE, FAKE, FAKE, FAKE, N, 4, 128, 128, N) == -1
    assert lib.fp8_gemm_rowscale(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 128, 192, N) == -2  # K % 128
    assert lib.fp8_gemm_rowscale(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 96, 128, N) == -2   # N % 128
    assert lib.fp8_gemm_rowscale(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 128, 128, N) == -1
    assert lib.attn_lse_merge(FAKE, FAKE, FAKE, FAKE, FAKE, N, 64, 1, 128, N) == -1
    assert lib.attn_lse_merge(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 1, 128, N) == -1
    assert lib.sol_attn_proxy_scores(FAKE, FAKE, FAKE, 60, 10, 64, 64, 1, 128, 64, N) == -1
    assert lib.sol_attn_block_mask(FAKE, FAKE, FAKE, FAKE, 0.0, 64, 10, 256, 256, 1, 128, 64,
                                   N, FAKE, N) == -1          # row0 not a multiple of 128
    assert lib.sol_attn_block_mask(FAKE, FAKE, FAKE, FAKE, math.nan, 0, 10, 256, 256, 1, 128,
                                   64, N, FAKE, N) == -1
    ts = lib.sol_attn_tile_schedule
    big = 1 << 40
    assert ts(FAKE, FAKE, FAKE, N, FAKE, 256, 1, 128, 128, 0.5, 0, FAKE, big, N) == -1  # no work
    assert ts(FAKE, FAKE, FAKE, FAKE, FAKE, 256, 1, 128, 128, -math.inf, 0, FAKE, big, N) == -1
    assert ts(FAKE, FAKE, FAKE, FAKE, FAKE, 256, 1, 128, 128, math.nan, 0, FAKE, big, N) == -1
    assert ts(FAKE, FAKE, FAKE, FAKE, FAKE, 256, 1, 128, 96, 0.5, 0, FAKE, big, N) == -2   # B
    assert ts(FAKE, FAKE, FAKE, FAKE, FAKE, 256, 1, 128, 128, 0.5, 0, FAKE, 16, N) == -1   # short ws
    assert ts(FAKE, FAKE, FAKE, FAKE, FAKE, 4097 * 128, 1, 128, 128, 0.5, 0, FAKE, big, N) == -2
    odd = ctypes.c_void_p(0x10002)  # not 4-byte aligned
    assert ts(FAKE, FAKE, FAKE, odd, FAKE, 256, 1, 128, 128, 0.5, 0, FAKE, big, N) == -1


def test_shard_entry_points_argument_errors(lib):
    N = None
    sh = lib.sol_attn_forward_shard
    need = lib.sol_attn_shard_workspace_size(256, 128, 4, 1, 128, 64, 0.5)
    assert need > 0
    # (q, k, v, kbar_all, part_o, part_ml, N, Nk, nb_all, H, d, B, beta, ws, ws_bytes, stream)
    assert sh(N, FAKE, FAKE, FAKE, FAKE, FAKE, 256, 128, 4, 1, 128, 64, 0.5, FAKE, need, N) == -1
    assert sh(FAKE, FAKE, FAKE, N, FAKE, FAKE, 256, 128, 4, 1, 128, 64, 0.5, FAKE, need, N) == -1  # no kbar_all
    assert sh(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 256, 128, 1, 1, 128, 64, 0.5, FAKE, need, N) == -1  # nb_all < local blocks
    assert sh(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 256, 0, 4, 1, 128, 64, 0.5, FAKE, need, N) == -1
    assert sh(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 256, 128, 4, 1, 128, 64, math.nan, FAKE, need, N) == -1
    assert sh(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 256, 128, 4, 1, 128, 64, 0.5, FAKE, need - 1, N) == -1
    assert sh(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 256, 128, 4, 1, 128, 48, 0.5, FAKE, need, N) == -2
    assert sh(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 256, 128, 4, 1, 64, 64, 0.5, FAKE, need, N) == -2
    # the dense share needs no pooled keys and no workspace
    assert lib.sol_attn_shard_workspace_size(256, 128, 0, 1, 128, 64, -math.inf) == 0
    cp = lib.sol_attn_combine_partials
    assert cp(FAKE, FAKE, 0, FAKE, N, 64, 1, 128, N) == -1      # S = 0
    assert cp(FAKE, N, 2, FAKE, N, 64, 1, 128, N) == -1
    assert cp(FAKE, FAKE, 2, FAKE, N, 64, 1, 96, N) == -2


def test_workspace_sizes(lib):
    ws = lib.sol_attn_workspace_size
    # 4K sequence: pooled K and V (fp32), bf16 block sums, mu and sigma -- O(H N + H nb d),
    # never the O(H N nb) proxy map
    H, N, B = 32, 130686, 128
    nb = (N + B - 1) // B
    s = ws(N, N, H, 128, B, 1)
    assert s >= 2 * H * nb * 128 * 4 + 2 * H * N * 4
    assert s < 128 * 2 ** 20  # pooled K/V, bf16 copies, mu, sigma: ~92 MB at 4K
    assert s < H * N * nb  # far below one byte per proxy score
    # dense self-attention at large N needs no workspace
    assert ws(N, N, H, 128, B, 0) == 0
    # short query against long keys: split partials
    assert ws(126, 130560, 32, 128, 128, 0) > 0
    assert ws(0, 10, 1, 128, 64, 1) == 0


def test_noalloc_argument_errors(lib):
    """The allocation-free forward checks its arguments like sol_attn_forward,
    then refuses a call needing more than its 128 MiB scratch -- all before
    any HIP call, so it runs without a GPU."""
    f = lib.sol_attn_forward_noalloc
    N = None
    assert f(N, FAKE, FAKE, FAKE, N, 64, 1, 128, 64, 0.0, 1, 0, N) == -1
    assert f(FAKE, FAKE, FAKE, FAKE, N, 0, 1, 128, 64, 0.0, 1, 0, N) == -1
    assert f(FAKE, FAKE, FAKE, FAKE, N, 64, 1, 64, 64, 0.0, 1, 0, N) == -2
    assert f(FAKE, FAKE, FAKE, FAKE, N, 64, 1, 128, 32, 0.0, 1, 0, N) == -2
    assert f(FAKE, FAKE, FAKE, FAKE, N, 64, 1, 128, 64, math.nan, 1, 0, N) == -1
    assert f(ctypes.c_void_p(0x10002), FAKE, FAKE, FAKE, N, 64, 1, 128, 64, 0.0, 1, 0, N) == -1
    # 64 heads x 140,000 tokens needs ~226 MiB of workspace
    assert lib.sol_attn_workspace_size(140000, 0, 64, 128, 128, 1) > 128 << 20
    assert f(FAKE, FAKE, FAKE, FAKE, N, 140000, 64, 128, 128, 0.5, 1, 0, N) == -4
    assert len(lib.sol_attn_error_string(-4)) > 0
    # the 4K latent workload fits
    assert lib.sol_attn_workspace_size(130686, 0, 32, 128, 128, 1) <= 128 << 20

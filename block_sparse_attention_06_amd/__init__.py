"""Python binding of libsolattn: MI355X (gfx950) query-thresholded block-sparse
attention with a Taylor term for rejected blocks (Sol-Attn style).

This module only marshals arguments: it checks shapes and dtypes, allocates
output tensors with torch, and calls the C ABI (``include/solattn.h``) on the
current HIP stream.  Every step of the computation runs in the HIP kernels of
``libsolattn.so``; there is no CPU or PyTorch fallback.  If the library is not
built, every call raises.

Tensors are torch tensors on the GPU, ``[H, N, 128]`` contiguous, bf16 for
q/k/v/out, fp32 for the rest.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

__all__ = [
    "SOL_DENSE",
    "SOL_SPARSE",
    "SolAttnError",
    "library_path",
    "load_library",
    "sol_attn_pool",
    "sol_attn_row_stats",
    "sol_attn_row_stats_moment",
    "sol_attn_forward",
    "sol_attn_forward_noalloc",
    "sol_attn_workspace_size",
    "attn_lse_merge",
    "sol_attn_error_string",
    "sol_attn_proxy_scores",
    "sol_attn_block_mask",
    "sol_attn_tile_schedule",
    "fp8_quantize_rows",
    "fp8_gemm_rowscale",
    "na3d_forward",
    "sol_attn_forward_shard",
    "sol_attn_shard_workspace_size",
    "sol_attn_combine_partials",
]

SOL_DENSE = 0
SOL_SPARSE = 1
HEAD_DIM = 128

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libsolattn.so"
_lib = None


class SolAttnError(RuntimeError):
    """A negative return code from the C ABI."""

    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed with code {code}: {sol_attn_error_string(code)}")
        self.code = code


def library_path() -> str:
    return os.path.join(_HERE, _LIB_NAME)


def load_library() -> ctypes.CDLL:
    """Load libsolattn.so from the package directory (built by ``build.py``)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m block_sparse_attention_06_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(path)
    P, I, F, S, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_char_p
    L = ctypes.c_int64
    sigs = {
        "sol_attn_pool": (I, [P, P, P, P, I, I, I, I, P]),
        "sol_attn_row_stats": (I, [P, P, P, P, I, I, I, I, I, P]),
        "sol_attn_row_stats_moment": (I, [P, P, P, P, I, I, I, I, I, P, S, P]),
        "sol_attn_forward": (I, [P, P, P, P, P, I, I, I, I, F, I, I, P, S, P]),
        "sol_attn_forward_noalloc": (I, [P, P, P, P, P, I, I, I, I, F, I, I, P]),
        "sol_attn_workspace_size": (S, [I, I, I, I, I, I]),
        "attn_lse_merge": (I, [P, P, P, P, P, P, I, I, I, P]),
        "sol_attn_error_string": (Z, [I]),
        "sol_attn_proxy_scores": (I, [P, P, P, I, I, I, I, I, I, I, P]),
        "sol_attn_block_mask": (I, [P, P, P, P, F, I, I, I, I, I, I, I, P, P, P]),
        "sol_attn_tile_schedule": (I, [P, P, P, P, P, I, I, I, I, F, I, P, S, P]),
        "fp8_quantize_rows": (I, [P, P, P, L, I, P]),
        "fp8_gemm_rowscale": (I, [P, P, P, P, P, I, I, I, P]),
        "na3d_forward": (I, [P, P, P, P, P, I, I, I, I, I, I, I, I, P]),
        "sol_attn_forward_shard": (I, [P, P, P, P, P, P, I, I, I, I, I, I, F, P, S, P]),
        "sol_attn_shard_workspace_size": (S, [I, I, I, I, I, I, F]),
        "sol_attn_combine_partials": (I, [P, P, I, P, P, I, I, I, P]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def sol_attn_error_string(code: int) -> str:
    return load_library().sol_attn_error_string(int(code)).decode()


def _check(fn: str, code: int) -> None:
    if code != 0:
        raise SolAttnError(fn, code)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _want(t: torch.Tensor, name: str, dtype: torch.dtype, ndim: int) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {ndim}-d tensor")


def _want_shape(t: torch.Tensor, name: str, dtype: torch.dtype, shape) -> None:
    """As _want, and the exact shape: the kernels index every buffer by the
    sizes passed alongside it, so a smaller tensor would be read or written
    out of bounds."""
    _want(t, name, dtype, len(shape))
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _want_ws(workspace: Optional[torch.Tensor]) -> int:
    """Bytes of a caller's workspace (device memory, contiguous), 0 if None."""
    if workspace is None:
        return 0
    if not isinstance(workspace, torch.Tensor) or not workspace.is_cuda:
        raise ValueError("workspace must be a GPU tensor")
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    return workspace.numel() * workspace.element_size()


def sol_attn_pool(k: torch.Tensor, v: torch.Tensor, B: int, stream=None):
    """Block means ``(kbar, vbar)`` ``[H, ceil(N/B), 128]`` fp32 of keys and values."""
    lib = load_library()
    _want(k, "k", torch.bfloat16, 3)
    _want_shape(v, "v", torch.bfloat16, k.shape)
    H, N, d = k.shape
    nb = (N + B - 1) // B
    kbar = torch.empty((H, nb, d), dtype=torch.float32, device=k.device)
    vbar = torch.empty_like(kbar)
    _check("sol_attn_pool", lib.sol_attn_pool(_ptr(k), _ptr(v), _ptr(kbar), _ptr(vbar),
                                              N, H, d, int(B), _stream(stream)))
    return kbar, vbar


def sol_attn_row_stats(q: torch.Tensor, kbar: torch.Tensor, B: int, Nk: int, stream=None):
    """``(mu, sigma)`` ``[H, N]`` fp32 of the block proxy scores of every query row."""
    lib = load_library()
    _want(q, "q", torch.bfloat16, 3)
    H, N, d = q.shape
    _want_shape(kbar, "kbar", torch.float32, (H, (int(Nk) + B - 1) // B, d))
    mu = torch.empty((H, N), dtype=torch.float32, device=q.device)
    sigma = torch.empty_like(mu)
    _check("sol_attn_row_stats", lib.sol_attn_row_stats(
        _ptr(q), _ptr(kbar), _ptr(mu), _ptr(sigma), N, int(Nk), H, d, int(B), _stream(stream)))
    return mu, sigma


def sol_attn_row_stats_moment(q: torch.Tensor, kbar: torch.Tensor, B: int, Nk: int,
                              workspace: Optional[torch.Tensor] = None, stream=None):
    """``(mu, sigma)`` as :func:`sol_attn_row_stats`, in moment form (the form the
    forward pass uses from 128 key blocks on).  ``workspace`` (uint8, at least
    ``H * (2*128*128*2 + 128*4 + 8*(128*128 + 2*128)*4)`` bytes) is allocated
    when not given."""
    lib = load_library()
    _want(q, "q", torch.bfloat16, 3)
    H, N, d = q.shape
    _want_shape(kbar, "kbar", torch.float32, (H, (int(Nk) + B - 1) // B, d))
    need = H * (2 * d * d * 2 + d * 4 + 8 * (d * d + 2 * d) * 4)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    have = _want_ws(workspace)
    mu = torch.empty((H, N), dtype=torch.float32, device=q.device)
    sigma = torch.empty_like(mu)
    _check("sol_attn_row_stats_moment", lib.sol_attn_row_stats_moment(
        _ptr(q), _ptr(kbar), _ptr(mu), _ptr(sigma), N, int(Nk), H, d, int(B),
        _ptr(workspace), have, _stream(stream)))
    return mu, sigma


def sol_attn_workspace_size(N: int, Nk: int, H: int, d: int, B: int, mode: int) -> int:
    return int(load_library().sol_attn_workspace_size(N, Nk, H, d, B, mode))


def sol_attn_forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, B: int = 128,
                     beta: float = 0.5, mode: int = SOL_SPARSE,
                     workspace: Optional[torch.Tensor] = None,
                     out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                     want_lse: bool = True, stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Attention forward; returns ``(out [H,N,128] bf16, lse [H,N] fp32 or None)``.

    ``workspace`` (uint8, at least ``sol_attn_workspace_size`` bytes) is allocated
    when not given; pass one to keep the call free of allocations."""
    lib = load_library()
    _want(q, "q", torch.bfloat16, 3)
    _want(k, "k", torch.bfloat16, 3)
    _want(v, "v", torch.bfloat16, 3)
    H, N, d = q.shape
    Nk = k.shape[1]
    if k.shape != v.shape or k.shape[0] != H or k.shape[2] != d:
        raise ValueError("k and v must be [H, Nk, d] with q's H and d")
    if out is None:
        out = torch.empty_like(q)
    else:
        _want(out, "out", torch.bfloat16, 3)
        if out.shape != q.shape:
            raise ValueError("out must have q's shape")
    if lse is None and want_lse:
        lse = torch.empty((H, N), dtype=torch.float32, device=q.device)
    elif lse is not None:
        _want_shape(lse, "lse", torch.float32, (H, N))
    ws_bytes = sol_attn_workspace_size(N, Nk, H, d, B, mode)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    have = _want_ws(workspace)
    if math.isnan(beta):
        raise ValueError("beta must not be NaN")
    _check("sol_attn_forward", lib.sol_attn_forward(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), N, H, d, int(B), float(beta),
        int(mode), Nk, _ptr(workspace), have, _stream(stream)))
    return out, lse


def sol_attn_tile_schedule(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, B: int = 128,
                           beta: float = 0.5, workspace: Optional[torch.Tensor] = None,
                           stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Work count ``[H, ceil(N/128)]`` int32 of every 128-row query tile and the
    order ``[H * ceil(N/128)]`` int32 (``h * n + t`` of the tile run r-th) in which
    a sparse :func:`sol_attn_forward` call of these sizes runs them when it orders
    its tiles."""
    lib = load_library()
    _want(q, "q", torch.bfloat16, 3)
    _want(k, "k", torch.bfloat16, 3)
    _want_shape(v, "v", torch.bfloat16, k.shape)
    H, N, d = q.shape
    Nk = k.shape[1]
    if k.shape[0] != H or k.shape[2] != d:
        raise ValueError("k and v must be [H, Nk, d] with q's H and d")
    if math.isnan(beta):
        raise ValueError("beta must not be NaN")
    n_qt = (N + 127) // 128
    work = torch.empty((H, n_qt), dtype=torch.int32, device=q.device)
    order = torch.empty((H * n_qt,), dtype=torch.int32, device=q.device)
    ws_bytes = sol_attn_workspace_size(N, Nk, H, d, B, SOL_SPARSE)
    if workspace is None:
        workspace = torch.empty(max(1, ws_bytes), dtype=torch.uint8, device=q.device)
    have = _want_ws(workspace)
    _check("sol_attn_tile_schedule", lib.sol_attn_tile_schedule(
        _ptr(q), _ptr(k), _ptr(v), _ptr(work), _ptr(order), N, H, d, int(B), float(beta), Nk,
        _ptr(workspace), have, _stream(stream)))
    return work, order


def sol_attn_forward_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                             out: torch.Tensor, lse: Optional[torch.Tensor] = None, B: int = 128,
                             beta: float = 0.5, mode: int = SOL_SPARSE, stream=None):
    """:func:`sol_attn_forward` for callers that cannot allocate: no workspace
    (the library's own per-GPU scratch, at most 128 MiB, is used) and no
    output allocated here -- ``out`` (and ``lse``, if wanted) must be given.
    Calls that overlap in time on one GPU share that scratch and race."""
    lib = load_library()
    _want(q, "q", torch.bfloat16, 3)
    _want(k, "k", torch.bfloat16, 3)
    _want(v, "v", torch.bfloat16, 3)
    H, N, d = q.shape
    Nk = k.shape[1]
    if k.shape != v.shape or k.shape[0] != H or k.shape[2] != d:
        raise ValueError("k and v must be [H, Nk, d] with q's H and d")
    _want_shape(out, "out", torch.bfloat16, (H, N, d))
    if lse is not None:
        _want_shape(lse, "lse", torch.float32, (H, N))
    if math.isnan(beta):
        raise ValueError("beta must not be NaN")
    _check("sol_attn_forward_noalloc", lib.sol_attn_forward_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), N, H, d, int(B), float(beta), int(mode),
        Nk, _stream(stream)))
    return out, lse


def attn_lse_merge(out_a: torch.Tensor, lse_a: torch.Tensor, out_b: torch.Tensor,
                   lse_b: torch.Tensor, out: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None, stream=None):
    """Exact merge of two partial answers over disjoint keys; returns ``(out, lse)``."""
    lib = load_library()
    _want(out_a, "out_a", torch.bfloat16, 3)
    H, N, d = out_a.shape
    _want_shape(out_b, "out_b", torch.bfloat16, (H, N, d))
    _want_shape(lse_a, "lse_a", torch.float32, (H, N))
    _want_shape(lse_b, "lse_b", torch.float32, (H, N))
    if out is None:
        out = torch.empty_like(out_a)
    _want_shape(out, "out", torch.bfloat16, (H, N, d))
    if lse is None:
        lse = torch.empty_like(lse_a)
    _want_shape(lse, "lse", torch.float32, (H, N))
    _check("attn_lse_merge", lib.attn_lse_merge(
        _ptr(out_a), _ptr(lse_a), _ptr(out_b), _ptr(lse_b), _ptr(out), _ptr(lse), N, H, d,
        _stream(stream)))
    return out, lse


def sol_attn_shard_workspace_size(N: int, Nk: int, nb_all: int, H: int, d: int, B: int,
                                  beta: float) -> int:
    return int(load_library().sol_attn_shard_workspace_size(N, Nk, nb_all, H, d, B,
                                                             float(beta)))


def sol_attn_forward_shard(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                           kbar_all: Optional[torch.Tensor], B: int = 128, beta: float = 0.5,
                           part_o: Optional[torch.Tensor] = None,
                           part_ml: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None, stream=None):
    """One rank's share of key-sharded Sol-Attn: the partial answer of every
    query row over the key blocks in ``k``/``v`` (whole blocks of the full
    sequence), with thresholds from ``kbar_all`` ``[H, nb_all, 128]`` (the
    pooled keys of every block).  Returns ``(part_o [H,N,128] fp32,
    part_ml [H,N,2] fp32)``; merge shares with :func:`sol_attn_combine_partials`."""
    lib = load_library()
    _want(q, "q", torch.bfloat16, 3)
    _want(k, "k", torch.bfloat16, 3)
    _want(v, "v", torch.bfloat16, 3)
    H, N, d = q.shape
    Nk = k.shape[1]
    if k.shape != v.shape or k.shape[0] != H or k.shape[2] != d:
        raise ValueError("k and v must be [H, Nk, d] with q's H and d")
    if math.isnan(beta):
        raise ValueError("beta must not be NaN")
    nb_all = 0
    if kbar_all is not None:
        _want(kbar_all, "kbar_all", torch.float32, 3)
        nb_all = kbar_all.shape[1]
        _want_shape(kbar_all, "kbar_all", torch.float32, (H, nb_all, d))
    if part_o is None:
        part_o = torch.empty((H, N, d), dtype=torch.float32, device=q.device)
    if part_ml is None:
        part_ml = torch.empty((H, N, 2), dtype=torch.float32, device=q.device)
    _want_shape(part_o, "part_o", torch.float32, (H, N, d))
    _want_shape(part_ml, "part_ml", torch.float32, (H, N, 2))
    ws_bytes = sol_attn_shard_workspace_size(N, Nk, nb_all, H, d, B, beta)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    have = _want_ws(workspace)
    _check("sol_attn_forward_shard", lib.sol_attn_forward_shard(
        _ptr(q), _ptr(k), _ptr(v), _ptr(kbar_all), _ptr(part_o), _ptr(part_ml), N, Nk, nb_all,
        H, d, int(B), float(beta), _ptr(workspace), have, _stream(stream)))
    return part_o, part_ml


def sol_attn_combine_partials(part_o: torch.Tensor, part_ml: torch.Tensor,
                              out: Optional[torch.Tensor] = None, want_lse: bool = True,
                              stream=None):
    """Exact merge of S partial answers ``part_o [S,H,N,128]``, ``part_ml [S,H,N,2]``
    (fp32); returns ``(out [H,N,128] bf16, lse [H,N] fp32 or None)``."""
    lib = load_library()
    _want(part_o, "part_o", torch.float32, 4)
    _want(part_ml, "part_ml", torch.float32, 4)
    S, H, N, d = part_o.shape
    if tuple(part_ml.shape) != (S, H, N, 2):
        raise ValueError("part_ml must be [S, H, N, 2]")
    if out is None:
        out = torch.empty((H, N, d), dtype=torch.bfloat16, device=part_o.device)
    _want_shape(out, "out", torch.bfloat16, (H, N, d))
    lse = torch.empty((H, N), dtype=torch.float32, device=part_o.device) if want_lse else None
    _check("sol_attn_combine_partials", lib.sol_attn_combine_partials(
        _ptr(part_o), _ptr(part_ml), S, _ptr(out), _ptr(lse), N, H, d, _stream(stream)))
    return out, lse


def sol_attn_proxy_scores(q: torch.Tensor, kbar: torch.Tensor, B: int, Nk: int,
                          row0: int = 0, nrows: Optional[int] = None, stream=None):
    """Proxy scores ``[H, nrows, nb]`` fp32 as the forward kernel computes them."""
    lib = load_library()
    _want(q, "q", torch.bfloat16, 3)
    H, N, d = q.shape
    nrows = N - row0 if nrows is None else nrows
    if row0 < 0 or nrows < 0 or row0 + nrows > N:
        raise ValueError("rows [row0, row0 + nrows) must lie within [0, N)")
    nb = (Nk + B - 1) // B
    _want_shape(kbar, "kbar", torch.float32, (H, nb, d))
    p = torch.empty((H, nrows, nb), dtype=torch.float32, device=q.device)
    _check("sol_attn_proxy_scores", lib.sol_attn_proxy_scores(
        _ptr(q), _ptr(kbar), _ptr(p), int(row0), int(nrows), N, int(Nk), H, d, int(B),
        _stream(stream)))
    return p


def sol_attn_block_mask(q: torch.Tensor, kbar: torch.Tensor, mu: torch.Tensor,
                        sigma: torch.Tensor, beta: float, B: int, Nk: int, row0: int = 0,
                        nrows: Optional[int] = None, want_mask: bool = True, stream=None):
    """Selection mask ``[H, nrows, nb]`` uint8 (or None) and the four density counts
    (selected pairs, 32-row tile pairs, 128-row tile pairs, 128-row tile total)."""
    lib = load_library()
    _want(q, "q", torch.bfloat16, 3)
    H, N, d = q.shape
    nrows = N - row0 if nrows is None else nrows
    if row0 < 0 or nrows < 0 or row0 + nrows > N:
        raise ValueError("rows [row0, row0 + nrows) must lie within [0, N)")
    nb = (Nk + B - 1) // B
    _want_shape(kbar, "kbar", torch.float32, (H, nb, d))
    _want_shape(mu, "mu", torch.float32, (H, N))
    _want_shape(sigma, "sigma", torch.float32, (H, N))
    mask = torch.empty((H, nrows, nb), dtype=torch.uint8, device=q.device) if want_mask else None
    counts = torch.empty(4, dtype=torch.int64, device=q.device)
    _check("sol_attn_block_mask", lib.sol_attn_block_mask(
        _ptr(q), _ptr(kbar), _ptr(mu), _ptr(sigma), float(beta), int(row0), int(nrows), N,
        int(Nk), H, d, int(B), _ptr(mask), _ptr(counts), _stream(stream)))
    return mask, counts


def fp8_quantize_rows(x: torch.Tensor, q: Optional[torch.Tensor] = None,
                      scale: Optional[torch.Tensor] = None, stream=None):
    """Per-row E4M3 quantisation of a bf16 ``[M, K]`` matrix: returns
    ``(codes [M, K] uint8, scale [M] fp32)`` with ``x ~ scale[:, None] * dec(codes)``;
    pass ``q`` and ``scale`` to write into existing tensors."""
    lib = load_library()
    _want(x, "x", torch.bfloat16, 2)
    M, K = x.shape
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty((M,), dtype=torch.float32, device=x.device)
    _want(q, "q", torch.uint8, 2)
    _want(scale, "scale", torch.float32, 1)
    if tuple(q.shape) != (M, K) or scale.shape[0] != M:
        raise ValueError("fp8_quantize_rows: output shape mismatch")
    _check("fp8_quantize_rows", lib.fp8_quantize_rows(_ptr(x), _ptr(q), _ptr(scale), M, K,
                                                      _stream(stream)))
    return q, scale


def fp8_gemm_rowscale(a: torch.Tensor, sa: torch.Tensor, w: torch.Tensor, sw: torch.Tensor,
                      out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """``y [M, N] bf16 = sa[:, None] * sw[None, :] * (dec(a) @ dec(w).T)`` with E4M3
    codes ``a [M, K]``, ``w [N, K]`` (uint8) and fp32 accumulation."""
    lib = load_library()
    _want(a, "a", torch.uint8, 2)
    _want(w, "w", torch.uint8, 2)
    _want(sa, "sa", torch.float32, 1)
    _want(sw, "sw", torch.float32, 1)
    M, K = a.shape
    N = w.shape[0]
    if w.shape[1] != K or sa.shape[0] != M or sw.shape[0] != N:
        raise ValueError("fp8_gemm_rowscale: shape mismatch")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    _want_shape(out, "out", torch.bfloat16, (M, N))
    _check("fp8_gemm_rowscale", lib.fp8_gemm_rowscale(_ptr(a), _ptr(sa), _ptr(w), _ptr(sw),
                                                      _ptr(out), M, N, K, _stream(stream)))
    return out


def na3d_forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, grid, window,
                 out: Optional[torch.Tensor] = None, want_lse: bool = True, stream=None):
    """3D neighbourhood attention: ``q, k, v [H, T*Y*X, 128]`` bf16 on the grid
    ``(T, Y, X)``, window ``(kt, ky, kx)`` (odd); returns ``(out, lse or None)``."""
    lib = load_library()
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _want(t, nm, torch.bfloat16, 3)
    H, n, d = q.shape
    T, Y, X = (int(x) for x in grid)
    kt, ky, kx = (int(x) for x in window)
    if n != T * Y * X or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("na3d_forward: shapes do not match the grid")
    if out is None:
        out = torch.empty_like(q)
    _want_shape(out, "out", torch.bfloat16, (H, n, d))
    lse = torch.empty((H, n), dtype=torch.float32, device=q.device) if want_lse else None
    _check("na3d_forward", lib.na3d_forward(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse) if lse is not None else None,
        T, Y, X, H, d, kt, ky, kx, _stream(stream)))
    return out, lse

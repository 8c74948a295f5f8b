"""The allocation-free forward entry point (sol_attn_forward_noalloc) through
the C ABI: its results equal, bit for bit, those of sol_attn_forward with a
caller workspace (the same kernels on the same plan), on two calls in a row
with the second smaller -- the library's scratch then still holds the first
call's contents, which the second must not read.  The workspace of the
reference calls is filled with 0xFF bytes (NaN in every float format) so that
a read of an unwritten workspace byte would show in the reference too.

Cases: sparse (157 key blocks, moment-form statistics, ragged last block) then
sparse (24 blocks, direct-form statistics); sparse with 2,048 query tiles, which
the call runs in order of decreasing work, then a small one; dense short-query
split-KV with its combine, then a smaller one.  Last, both cases captured into one HIP graph
and replayed with eager calls of other sizes in between."""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import block_sparse_attention_06_amd as sa  # noqa: E402
from synth import Workload, clustered, gaussian  # noqa: E402
from tests.parity_utils import check_close, dev, host  # noqa: E402

pytestmark = pytest.mark.gpu


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _with_workspace(lib, q, k, v, B, beta, mode):
    H, N, d = q.shape
    Nk = k.shape[1]
    nbytes = lib.sol_attn_workspace_size(N, Nk, H, d, B, mode)
    ws = torch.full((max(1, nbytes),), 0xFF, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty((H, N), dtype=torch.float32, device="cuda")
    r = lib.sol_attn_forward(_p(q), _p(k), _p(v), _p(out), _p(lse), N, H, d, B, beta, mode, Nk,
                             _p(ws), nbytes, _stream())
    assert r == 0, sa.sol_attn_error_string(r)
    return out, lse


def _noalloc(lib, q, k, v, B, beta, mode):
    H, N, d = q.shape
    Nk = k.shape[1]
    out = torch.full_like(q, float("nan"))
    lse = torch.full((H, N), float("nan"), dtype=torch.float32, device="cuda")
    r = lib.sol_attn_forward_noalloc(_p(q), _p(k), _p(v), _p(out), _p(lse), N, H, d, B, beta, mode,
                                     Nk, _stream())
    assert r == 0, sa.sol_attn_error_string(r)
    return out, lse


def _sparse_inputs(H, N, B, seed):
    w = Workload("noalloc", H, N, 0, 128, B, (N + B - 1) // B, 0.5, seed, (0.5,))
    Q, K, V = clustered(w)
    return dev(Q), dev(K), dev(V)


def _dense_inputs(H, nq, nk, seed):
    Q, K, V = gaussian(H, nq, 128, seed=seed, nk=nk)
    return dev(Q), dev(K), dev(V)


@pytest.mark.parametrize("case", ["sparse", "sparse_ordered", "dense_split"])
def test_noalloc_matches_workspace_call_twice(case):
    lib = sa.load_library()
    if case == "sparse":
        calls = [(_sparse_inputs(8, 20000, 128, 21), 128, 0.5, sa.SOL_SPARSE),
                 (_sparse_inputs(2, 3000, 128, 22), 128, 0.5, sa.SOL_SPARSE)]
    elif case == "sparse_ordered":  # 16 x 128 tiles: the call orders them (tile work and order in scratch)
        calls = [(_sparse_inputs(16, 16384, 128, 25), 128, 0.5, sa.SOL_SPARSE),
                 (_sparse_inputs(2, 3000, 128, 26), 128, 1.0, sa.SOL_SPARSE)]
    else:
        calls = [(_dense_inputs(16, 126, 40000, 23), 128, 0.0, sa.SOL_DENSE),
                 (_dense_inputs(4, 100, 9000, 24), 128, 0.0, sa.SOL_DENSE)]
    for i, ((q, k, v), B, beta, mode) in enumerate(calls):
        got_o, got_l = _noalloc(lib, q, k, v, B, beta, mode)
        ref_o, ref_l = _with_workspace(lib, q, k, v, B, beta, mode)
        torch.cuda.synchronize()
        check_close(host(got_o).reshape(-1, 128), host(ref_o).reshape(-1, 128),
                    host(got_l).ravel(), host(ref_l).ravel(), what=f"{case} call {i}")
        assert torch.equal(got_o, ref_o) and torch.equal(got_l, ref_l), f"{case} call {i}"
        assert np.isfinite(host(ref_o)).all()


def test_noalloc_rejects_oversized_call():
    """A call needing more than the 128 MiB scratch is refused before any launch."""
    lib = sa.load_library()
    H, N = 64, 140000
    assert lib.sol_attn_workspace_size(N, N, H, 128, 128, sa.SOL_SPARSE) > 128 << 20
    q = torch.empty((1, 1, 128), dtype=torch.bfloat16, device="cuda")  # never read
    r = lib.sol_attn_forward_noalloc(_p(q), _p(q), _p(q), _p(q), None, N, H, 128, 128, 0.5,
                                     sa.SOL_SPARSE, N, _stream())
    assert r == -4, r


def test_noalloc_replays_in_a_graph():
    """Callers that cannot allocate are typically under graph capture: the
    entry point, set up by one eager call, captures kernels only, and every
    replay equals the eager result bit for bit although eager calls of other
    sizes use the same scratch between the replays."""
    lib = sa.load_library()
    sp = (_sparse_inputs(4, 3000, 128, 31), 128, 0.5, sa.SOL_SPARSE)
    dn = (_dense_inputs(8, 100, 20000, 32), 128, 0.0, sa.SOL_DENSE)
    others = [(_sparse_inputs(2, 2500, 128, 33), 128, 0.5, sa.SOL_SPARSE),
              (_dense_inputs(16, 126, 30000, 34), 128, 0.0, sa.SOL_DENSE)]
    eager = [_noalloc(lib, *qkv, B, beta, mode) for qkv, B, beta, mode in (sp, dn)]
    torch.cuda.synchronize()

    outs = []
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for (q, k, v), B, beta, mode in (sp, dn):
            H, N, d = q.shape
            out = torch.empty_like(q)
            lse = torch.empty((H, N), dtype=torch.float32, device="cuda")
            r = lib.sol_attn_forward_noalloc(_p(q), _p(k), _p(v), _p(out), _p(lse), N, H, d, B,
                                             beta, mode, k.shape[1], _stream())
            assert r == 0, sa.sol_attn_error_string(r)
            outs.append((out, lse))
    torch.cuda.synchronize()

    for rep in range(4):
        for o, l in outs:
            o.fill_(float("nan"))
            l.fill_(float("nan"))
        # eager work between replays leaves other contents in the scratch
        qkv, B, beta, mode = others[rep % 2]
        _noalloc(lib, *qkv, B, beta, mode)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, ((o, l), (ro, rl)) in enumerate(zip(outs, eager)):
            assert torch.equal(o, ro) and torch.equal(l, rl), f"replay {rep}: call {i}"

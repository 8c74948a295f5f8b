"""Concurrent calls on two streams of the same GPU.

doubleAI page "LTX-2.5 at 4K, in half the time", section "Inside the decoder":
a kernel that reset a shared synchronisation state too early produced wrong
results only when other work shared the GPU.  The hot-path kernels keep all
synchronisation inside a workgroup (barriers and LDS) and write only their own
outputs and workspace, so calls on different streams that write disjoint
buffers may overlap (the header's contract).  This checks that claim: the
sparse call (moment-form statistics, ragged last block) and a split-KV dense
short-query call with its combine run on two default-priority streams at
once, each with its own workspace and outputs, several times over, and every
result must equal, bit for bit, the same call run alone.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import block_sparse_attention_06_amd as sa  # noqa: E402
from synth import Workload, clustered, gaussian  # noqa: E402
from tests.parity_utils import dev  # noqa: E402

pytestmark = pytest.mark.gpu


def _inputs():
    # 16 heads x 20,000 tokens, 157 key blocks of 128 (the last one ragged):
    # moment-form statistics, 2,512 sparse workgroups
    H, N, B = 16, 20000, 128
    w = Workload("streams", H, N, 0, 128, B, (N + B - 1) // B, 0.5, 11, (0.5,))
    Q, K, V = clustered(w, threads=8)
    sparse = dict(q=dev(Q), k=dev(K), v=dev(V), B=B, beta=0.5)
    # short query set against many keys: keys split over workgroups + combine
    Qc, Kc, Vc = gaussian(16, 126, 128, seed=12, nk=40000)
    dense = dict(q=dev(Qc), k=dev(Kc), v=dev(Vc))
    return sparse, dense


def _run_sparse(c, ws, out, lse, stream):
    sa.sol_attn_forward(c["q"], c["k"], c["v"], B=c["B"], beta=c["beta"], mode=sa.SOL_SPARSE,
                        workspace=ws, out=out, lse=lse, stream=stream)


def _run_dense(c, ws, out, lse, stream):
    sa.sol_attn_forward(c["q"], c["k"], c["v"], mode=sa.SOL_DENSE, workspace=ws, out=out,
                        lse=lse, stream=stream)


def _buffers(c, mode, B=128):
    H, N, d = c["q"].shape
    Nk = c["k"].shape[1]
    ws = torch.empty(max(1, sa.sol_attn_workspace_size(N, Nk, H, d, B, mode)), dtype=torch.uint8,
                     device="cuda")
    return ws, torch.empty_like(c["q"]), torch.empty((H, N), dtype=torch.float32, device="cuda")


def test_two_streams_bitwise_equal_to_serial():
    sparse, dense = _inputs()
    main = torch.cuda.current_stream()
    # serial references, one call at a time
    ws_s, ref_os, ref_ls = _buffers(sparse, sa.SOL_SPARSE)
    ws_d, ref_od, ref_ld = _buffers(dense, sa.SOL_DENSE)
    _run_sparse(sparse, ws_s, ref_os, ref_ls, main)
    torch.cuda.synchronize()
    _run_dense(dense, ws_d, ref_od, ref_ld, main)
    torch.cuda.synchronize()

    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()  # default priority
    pairs = [(_buffers(sparse, sa.SOL_SPARSE), _buffers(dense, sa.SOL_DENSE)) for _ in range(2)]
    another = _buffers(sparse, sa.SOL_SPARSE)
    for rep in range(3):
        for (bs, bd) in pairs:
            for t in (*bs, *bd):
                if t.dtype != torch.uint8:
                    t.fill_(float("nan"))
        for t in another[1:]:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        # two sparse calls and two split-KV dense calls in flight on two streams
        _run_sparse(sparse, *pairs[0][0], s1)
        _run_sparse(sparse, *another, s2)
        _run_dense(dense, *pairs[0][1], s2)
        _run_dense(dense, *pairs[1][1], s1)
        _run_sparse(sparse, *pairs[1][0], s2)
        torch.cuda.synchronize()
        for i, (bs, bd) in enumerate(pairs):
            assert torch.equal(bs[1], ref_os) and torch.equal(bs[2], ref_ls), f"sparse {i} rep {rep}"
            assert torch.equal(bd[1], ref_od) and torch.equal(bd[2], ref_ld), f"dense {i} rep {rep}"
        assert torch.equal(another[1], ref_os) and torch.equal(another[2], ref_ls)
    assert np.isfinite(ref_os.float().cpu().numpy()).all()

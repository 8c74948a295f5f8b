"""The library's calls under HIP graph capture: every entry point used on the
hot path enqueues kernels only (no allocation, no memset, no synchronisation;
the sparse calls include one large enough to order its query tiles),
so a captured sequence replays to the eager results bit for bit.  The graph
is replayed several times with eager work and synchronisations in between,
and every replay is checked (the kernels are deterministic)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import block_sparse_attention_06_amd as sa  # noqa: E402
from synth import clustered_head, gaussian  # noqa: E402
from tests.parity_utils import dev  # noqa: E402

pytestmark = pytest.mark.gpu


def _clustered(H, n, B, centres, seed):
    Q = np.empty((H, n, 128), np.uint16)
    K, V = np.empty_like(Q), np.empty_like(Q)
    for h in range(H):
        Q[h], K[h], V[h] = clustered_head(n, 128, B, centres, 0.5, seed, h)
    return Q, K, V


def test_hot_path_replays_in_a_graph():
    H, N, B = 4, 3000, 128
    Q, K, V = _clustered(H, N, B, 24, seed=21)
    q, k, v = dev(Q), dev(K), dev(V)
    # short queries against the same keys: split-KV inside the call, then the
    # two halves of the keys merged
    qs = q[:, :126].contiguous()
    half = 1536
    ka, kb_ = k[:, :half].contiguous(), k[:, half:].contiguous()
    va, vb = v[:, :half].contiguous(), v[:, half:].contiguous()
    kbar_all, _ = sa.sol_attn_pool(k, v, B)
    # 16 heads x 128 query tiles: the call runs its tiles in order of decreasing work
    Qo, Ko, Vo = _clustered(16, 16384, B, 128, seed=23)
    qo, ko, vo = dev(Qo), dev(Ko), dev(Vo)
    ws_o = torch.empty(sa.sol_attn_workspace_size(16384, 16384, 16, 128, B, sa.SOL_SPARSE),
                       dtype=torch.uint8, device="cuda")
    grid = (4, 12, 20)
    Qn, Kn, Vn = gaussian(2, int(np.prod(grid)), 128, seed=22)
    qn, kn, vn = dev(Qn), dev(Kn), dev(Vn)

    def buffers():
        f32, bf = torch.float32, torch.bfloat16
        return dict(
            o_sp=torch.empty_like(q), l_sp=torch.empty((H, N), dtype=f32, device="cuda"),
            o_or=torch.empty_like(qo), l_or=torch.empty((16, 16384), dtype=f32, device="cuda"),
            o_dn=torch.empty_like(q), l_dn=torch.empty((H, N), dtype=f32, device="cuda"),
            o_a=torch.empty_like(qs), l_a=torch.empty((H, 126), dtype=f32, device="cuda"),
            o_b=torch.empty_like(qs), l_b=torch.empty((H, 126), dtype=f32, device="cuda"),
            o_m=torch.empty_like(qs), l_m=torch.empty((H, 126), dtype=f32, device="cuda"),
            p_o=torch.empty((2, H, N, 128), dtype=f32, device="cuda"),
            p_ml=torch.empty((2, H, N, 2), dtype=f32, device="cuda"),
            o_sh=torch.empty_like(q),
            o_na=torch.empty_like(qn),
        )

    ws = torch.empty(sa.sol_attn_workspace_size(N, N, H, 128, B, sa.SOL_SPARSE),
                     dtype=torch.uint8, device="cuda")
    ws_a = torch.empty(max(1, sa.sol_attn_workspace_size(126, half, H, 128, B, sa.SOL_DENSE)),
                       dtype=torch.uint8, device="cuda")
    ws_b = torch.empty(max(1, sa.sol_attn_workspace_size(126, N - half, H, 128, B, sa.SOL_DENSE)),
                       dtype=torch.uint8, device="cuda")
    cut = 12 * B
    ws_s = [torch.empty(max(1, sa.sol_attn_shard_workspace_size(N, n_k, kbar_all.shape[1], H, 128,
                                                                B, 0.5)),
                        dtype=torch.uint8, device="cuda") for n_k in (cut, N - cut)]
    shards = [(k[:, :cut].contiguous(), v[:, :cut].contiguous()),
              (k[:, cut:].contiguous(), v[:, cut:].contiguous())]

    def run(b):
        sa.sol_attn_forward(q, k, v, B=B, beta=0.5, workspace=ws, out=b["o_sp"], lse=b["l_sp"])
        sa.sol_attn_forward(qo, ko, vo, B=B, beta=0.5, workspace=ws_o, out=b["o_or"],
                            lse=b["l_or"])
        sa.sol_attn_forward(q, k, v, mode=sa.SOL_DENSE, workspace=ws, out=b["o_dn"],
                            lse=b["l_dn"])
        sa.sol_attn_forward(qs, ka, va, mode=sa.SOL_DENSE, workspace=ws_a, out=b["o_a"],
                            lse=b["l_a"])
        sa.sol_attn_forward(qs, kb_, vb, mode=sa.SOL_DENSE, workspace=ws_b, out=b["o_b"],
                            lse=b["l_b"])
        sa.attn_lse_merge(b["o_a"], b["l_a"], b["o_b"], b["l_b"], out=b["o_m"], lse=b["l_m"])
        for s, (ks, vs) in enumerate(shards):
            sa.sol_attn_forward_shard(q, ks, vs, kbar_all, B=B, beta=0.5, part_o=b["p_o"][s],
                                      part_ml=b["p_ml"][s], workspace=ws_s[s])
        sa.sol_attn_combine_partials(b["p_o"], b["p_ml"], out=b["o_sh"], want_lse=False)
        sa.na3d_forward(qn, kn, vn, grid, (3, 5, 7), out=b["o_na"], want_lse=False)

    eager = buffers()
    run(eager)
    torch.cuda.synchronize()

    graphed = buffers()
    run(graphed)  # warm-up on the side stream torch captures on is not needed: one eager pass
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(graphed)
    torch.cuda.synchronize()

    for rep in range(4):
        for t in graphed.values():
            t.zero_()
        # eager work of the program between replays
        sa.sol_attn_forward(q, k, v, B=B, beta=1.0, workspace=ws, out=eager["o_dn"].clone())
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, ref in eager.items():
            got = graphed[name]
            assert torch.equal(got, ref), f"replay {rep}: {name} differs from the eager result"

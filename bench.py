#!/usr/bin/env python3
"""Benchmark of the block-sparse attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  * 4K Stage-2 self-attention, query-thresholded block-sparse with the Taylor
    term (pool + row statistics + fused forward, one sol_attn_forward call):
    H=32, N=130,686 (130,560 video + 126 audio tokens), d=128, B=128, beta=0.5;
  * audio->video cross-attention, dense: 126 queries against the two halves of
    130,560 video keys (65,280 each, split-KV inside each call) and the exact
    LSE merge of the two partial answers.
Inputs are resident in HBM before timing starts.  The metric is ms/call and
dense-equivalent TFLOP/s (4 H N^2 d for self-attention, 4 H Nq Nk d for
cross-attention) against the bf16 MFMA peak.

Prints one JSON line.  Only one GPU is used; --gpus above 1 exits.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk)
PEAK_FP8_TFLOPS = 5033.2    # MI355X dense fp8 MFMA (twice the bf16 rate)
PEAK_HBM_GBS = 8000.0
# a sparse call without a key split orders its query tiles from this many tiles
# in all, with at most ORDER_MAX_TILES per head (the library's launch rule)
ORDER_MIN_TILES = 2048
ORDER_MAX_TILES = 4096
METRIC = "ms/call + dense-equivalent TFLOP/s (% bf16 MFMA peak), 4K Stage-2 sparse attention"
KERNEL_SOURCES = ["block_sparse_attention_06_amd/csrc/forward.hip",
                  "block_sparse_attention_06_amd/csrc/device.hpp"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fwd_sparse_4k_beta0.5_traffic.json")


def kernel_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--beta", type=float, default=0.5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extras", action="store_true", help="skip beta=1.0 and dense 4K lines")
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="approximate CPU time budget of the oracle baseline sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run three plain 1 GiB device-to-device copies (reference "
                         "kernel of known traffic for hardware byte counters)")
    return ap.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def cpu_baseline(Q, K, V, B, beta, budget_s):
    """The fp64 oracle (as is) on a bounded, deterministic sample: whole
    128-row query tiles -- the first, middle and last of each head in turn --
    until about ``budget_s`` seconds of CPU work.  Reported in the same unit,
    dense-equivalent TFLOP/s, and extrapolated to the whole call."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    H, N, d = Q.shape
    nqt = (N + 127) // 128
    sample = [(h, t) for h in range(H) for t in (0, nqt // 2, nqt - 1)]
    done_rows = 0
    tiles = []
    t0 = time.perf_counter()
    for h, t in sample:
        if time.perf_counter() - t0 >= budget_s:
            break
        rows = np.arange(t * 128, min(N, (t + 1) * 128))
        q, k, v = (O.bf16_to_f64(x[h]) for x in (Q, K, V))
        O.sol_attn_head_ref(q, k, v, B, beta, rows=rows)
        done_rows += len(rows)
        tiles.append((h, t))
    el = time.perf_counter() - t0
    flops = 4.0 * done_rows * N * d
    full_s = el * (H * N) / done_rows
    return {
        "value": flops / el / 1e12,
        "unit": "TFLOP/s (dense-equivalent)",
        "cores": int(cores),
        "kind": "oracle",
        "sample": f"{len(tiles)} 128-row query tiles of the 4K workload (first, middle and last "
                  f"tile of heads 0..{tiles[-1][0]}), beta={beta}, fp64 numpy, {el:.1f} s wall",
        "ms_per_call_extrapolated": full_s * 1e3,
    }


def cpu_full_calls(gpu_ms):
    """The fp64 oracle (as is) on whole calls of the small workloads, timed on
    the host beside the GPU: tiny (beta 0), stage-1 768x512 (beta 0.5) and one
    head of the audio->video cross-attention (dense).  ``gpu_ms`` maps each
    name to the GPU's ms/call of the same call (the cross head: a 32-head call
    divided by 32)."""
    import oracle as O
    from synth import CROSS, WORKLOADS, clustered, cross_head
    res = {}
    for name, beta in (("tiny", 0.0), ("stage1", 0.5)):
        w = WORKLOADS[name]
        Q, K, V = clustered(w, threads=16)
        t0 = time.perf_counter()
        O.sol_attn_ref(Q, K, V, w.block, beta)
        el = time.perf_counter() - t0
        flops = 4.0 * w.heads * w.n * w.n * w.head_dim
        res[f"{name}_beta{beta}"] = {
            "oracle_ms_per_call": el * 1e3, "oracle_tflops_dense_equiv": flops / el / 1e12,
            "gpu_ms_per_call": gpu_ms.get(name), "heads": w.heads, "tokens": w.n}
    c = CROSS
    q, k, v = cross_head(c["nq"], c["nk"], c["head_dim"], c["seed"], 0)
    t0 = time.perf_counter()
    O.dense_ref(q[None], k[None], v[None])
    el = time.perf_counter() - t0
    flops = 4.0 * c["nq"] * c["nk"] * c["head_dim"]
    res["cross_one_head"] = {"oracle_ms_per_call": el * 1e3,
                             "oracle_tflops_dense_equiv": flops / el / 1e12,
                             "gpu_ms_per_head": gpu_ms.get("cross_head"),
                             "queries": c["nq"], "keys": c["nk"]}
    return res


def fp8_projection(sa, torch, tokens, hidden, dev, stream, reps=5):
    """FP8 projection around attention at the 4K token count: per-row E4M3
    quantisation of bf16 activations [tokens, hidden], then the GEMM against
    E4M3 weights [hidden, hidden] with per-channel scales (synthetic N(0, 1)
    activations and N(0, 1/hidden) weights)."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    x = torch.randn((tokens, hidden), generator=gen, device=dev).to(torch.bfloat16)
    wt = (torch.randn((hidden, hidden), generator=gen, device=dev) * hidden ** -0.5).to(torch.bfloat16)
    wq, wsc = sa.fp8_quantize_rows(wt)
    aq = torch.empty((tokens, hidden), dtype=torch.uint8, device=dev)
    asc = torch.empty((tokens,), dtype=torch.float32, device=dev)
    y = torch.empty((tokens, hidden), dtype=torch.bfloat16, device=dev)
    sa.fp8_quantize_rows(x, q=aq, scale=asc)
    sa.fp8_gemm_rowscale(aq, asc, wq, wsc, out=y)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ev[0].record(stream)
    for _ in range(reps):
        sa.fp8_quantize_rows(x, q=aq, scale=asc)
    ev[1].record(stream)
    for _ in range(reps):
        sa.fp8_gemm_rowscale(aq, asc, wq, wsc, out=y)
    ev[2].record(stream)
    torch.cuda.synchronize()
    q_ms = ev[0].elapsed_time(ev[1]) / reps
    g_ms = ev[1].elapsed_time(ev[2]) / reps
    flops = 2.0 * tokens * hidden * hidden
    q_bytes = tokens * hidden * (2 + 1) + tokens * 4  # bf16 read once, codes + scales written
    return {"tokens": tokens, "in_features": hidden, "out_features": hidden,
            "quantize_ms": q_ms, "quantize_gbs": q_bytes / q_ms / 1e6,
            "gemm_ms": g_ms, "gemm_tflops": flops / g_ms / 1e9,
            "pct_fp8_peak": 100 * flops / g_ms / 1e9 / PEAK_FP8_TFLOPS}


def workload_lines(sa, torch, name, to_dev, stream, reps=5, per_token=False):
    """ms/call, dense-equivalent TFLOP/s and achieved densities of one of the
    smaller latent workloads (same clustered generator), per beta; with
    ``per_token`` the generator's stress variant (one query centre per token)."""
    from synth import WORKLOADS, clustered
    w = WORKLOADS[name]
    H, N, d, B = w.heads, w.n, w.head_dim, w.block
    Q, K, V = clustered(w, threads=16, per_token=per_token)
    q, k, v = to_dev(Q), to_dev(K), to_dev(V)
    out = torch.empty_like(q)
    lse = torch.empty((H, N), dtype=torch.float32, device=q.device)
    ws = torch.empty(max(1, sa.sol_attn_workspace_size(N, N, H, d, B, sa.SOL_SPARSE)),
                     dtype=torch.uint8, device=q.device)
    kb, _ = sa.sol_attn_pool(k, v, B)
    nb = (N + B - 1) // B
    # the statistics the call routes with (moment form from 128 blocks on)
    stats = sa.sol_attn_row_stats_moment if nb >= 128 else sa.sol_attn_row_stats
    mu, sigma = stats(q, kb, B, N)
    flops = 4.0 * H * N * N * d
    res = {"heads": H, "tokens": N, "block": B, "centres": w.centres, "seed": w.seed,
           "query_centres": "per token" if per_token else "per query block"}
    for beta in w.betas:
        mode = sa.SOL_DENSE if beta == float("-inf") else sa.SOL_SPARSE
        call = lambda: sa.sol_attn_forward(q, k, v, B=B, beta=beta, mode=mode, workspace=ws,
                                           out=out, lse=lse)
        call()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(reps):
            call()
        ev[1].record(stream)
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1]) / reps
        line = {"ms_per_call": ms, "dense_equiv_tflops": flops / ms / 1e9}
        if mode == sa.SOL_SPARSE:
            _, c = sa.sol_attn_block_mask(q, kb, mu, sigma, beta, B, N, want_mask=False)
            c = c.cpu().numpy()
            line.update(rho_row=c[0] / (H * N * nb), rho_tile32=c[1] / (H * ((N + 31) // 32) * nb),
                        rho_tile128=c[2] / c[3])
        res["beta_" + ("-inf" if beta == float("-inf") else str(beta))] = line
    del q, k, v, out, ws
    return res


def cross_unsplit(sa, torch, qc, ks, vs, stream, halves_ms, reps=10):
    """The audio->video cross-attention as one call over all video keys (the
    call splits the keys over workgroups and merges the partials itself),
    beside the two-halves-plus-merge form of the timed step.  HBM roofline:
    K and V read once."""
    k = torch.cat(ks, dim=1)
    v = torch.cat(vs, dim=1)
    H, nq, d = qc.shape
    nk = k.shape[1]
    out = torch.empty_like(qc)
    lse = torch.empty((H, nq), dtype=torch.float32, device=qc.device)
    ws = torch.empty(max(1, sa.sol_attn_workspace_size(nq, nk, H, d, 128, sa.SOL_DENSE)),
                     dtype=torch.uint8, device=qc.device)
    call = lambda: sa.sol_attn_forward(qc, k, v, mode=sa.SOL_DENSE, workspace=ws, out=out, lse=lse)
    call()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(reps):
        call()
    ev[1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / reps
    kv_bytes = 2.0 * H * nk * d * 2
    del k, v, ws
    return {"queries": nq, "keys": nk, "ms_per_call": ms, "halves_plus_merge_ms": halves_ms,
            "roofline": {"bound": "hbm", "achieved": kv_bytes / ms / 1e6, "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": kv_bytes / ms / 1e6 / PEAK_HBM_GBS,
                         "work": "K and V read once"}}


def kv_sharded(sa, torch, q, k, v, B, beta, stream, dense_flops, unsplit_ms, ranks=2, reps=3):
    """Key-sharded Sol-Attn at 4K on one GPU: each rank's share of whole key
    blocks (its keys against every query, thresholds from the pooled keys of
    every block), run one after another, and the exact merge of the shares.
    In a deployment each share runs on its own GPU; the exchange of pooled
    keys and partial answers is not timed here."""
    H, N, d = q.shape
    nb = (N + B - 1) // B
    cuts = [round(i * nb / ranks) for i in range(ranks + 1)]
    kbar_all, _ = sa.sol_attn_pool(k, v, B)
    shares = []
    for r in range(ranks):
        lo, hi = cuts[r] * B, min(N, cuts[r + 1] * B)
        shares.append((k[:, lo:hi].contiguous(), v[:, lo:hi].contiguous()))
    part_o = torch.empty((ranks, H, N, d), dtype=torch.float32, device=q.device)
    part_ml = torch.empty((ranks, H, N, 2), dtype=torch.float32, device=q.device)
    wss = [torch.empty(max(1, sa.sol_attn_shard_workspace_size(N, ks.shape[1], nb, H, d, B, beta)),
                       dtype=torch.uint8, device=q.device) for ks, _ in shares]
    out = torch.empty_like(q)

    def run(ev=None):
        for r, (ks, vs) in enumerate(shares):
            sa.sol_attn_forward_shard(q, ks, vs, kbar_all, B=B, beta=beta, part_o=part_o[r],
                                      part_ml=part_ml[r], workspace=wss[r])
            if ev is not None:
                ev[r + 1].record(stream)
        sa.sol_attn_combine_partials(part_o, part_ml, out=out)
        if ev is not None:
            ev[ranks + 1].record(stream)

    run()
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(ranks + 2)]
        ev[0].record(stream)
        run(ev)
        torch.cuda.synchronize()
        times.append([ev[i].elapsed_time(ev[i + 1]) for i in range(ranks + 1)])
    t = np.median(np.array(times), axis=0)
    return {"ranks": ranks, "blocks_per_rank": [cuts[r + 1] - cuts[r] for r in range(ranks)],
            "share_ms": [float(x) for x in t[:ranks]], "combine_ms": float(t[ranks]),
            "sum_ms": float(t.sum()), "unsplit_ms": unsplit_ms,
            "per_rank_dense_equiv_tflops": dense_flops / ranks / float(np.max(t[:ranks])) / 1e9}


def na3d_decoder_tile(sa, torch, dev, stream, reps=10):
    """3D neighbourhood attention over one decoder tile of four latent frames
    of the 4K grid (4 x 68 x 120 tokens), 16 heads of 128, window 3 x 7 x 7
    (synthetic N(0, 1) bf16).  Algorithmic bytes: q, k, v read once, out and
    lse written once; algorithmic flops 4 d per (query, window key)."""
    T, Y, X, H, d = 4, 68, 120, 16, 128
    kt, ky, kx = 3, 7, 7
    n = T * Y * X
    gen = torch.Generator(device=dev)
    gen.manual_seed(6)
    q, k, v = (torch.randn((H, n, d), generator=gen, device=dev).to(torch.bfloat16)
               for _ in range(3))
    out = torch.empty_like(q)
    sa.na3d_forward(q, k, v, (T, Y, X), (kt, ky, kx), out=out)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(reps):
        sa.na3d_forward(q, k, v, (T, Y, X), (kt, ky, kx), out=out)
    ev[1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / reps
    alg_bytes = H * n * (4 * d * 2 + 4)
    alg_flops = 4.0 * d * kt * ky * kx * H * n
    # keys multiplied on the matrix core: a wave of 32 queries (4 rows x 8
    # columns of one frame) multiplies, in each of its kt key frames, the
    # 3 + ky key rows of its patch in pairs of 16-column rows
    exec_flops = 4.0 * d * kt * ((3 + ky + 1) // 2) * 32 * H * n
    achieved = alg_bytes / ms / 1e6
    return {"grid": [T, Y, X], "window": [kt, ky, kx], "heads": H, "head_dim": d,
            "ms": ms, "alg_tflops": alg_flops / ms / 1e9,
            "executed_mfma_tflops": exec_flops / ms / 1e9,
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS}}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); multi-GPU runs "
              "are out of scope for this library", file=sys.stderr)
        sys.exit(2)
    import torch

    import block_sparse_attention_06_amd as sa
    from synth import CROSS, WORKLOADS, clustered, cross

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def to_dev(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)

    w = WORKLOADS["4k"]
    H, N, d, B = w.heads, w.n, w.head_dim, w.block
    log(f"generating 4K inputs H={H} N={N}")
    Q, K, V = clustered(w, threads=16)
    q, k, v = to_dev(Q), to_dev(K), to_dev(V)
    c = CROSS
    log("generating cross-attention inputs")
    Qc, Kc, Vc = cross(c["heads"], c["nq"], c["nk"], c["head_dim"], c["seed"], threads=16)
    qc = to_dev(Qc)
    s = c["split"]
    kca, kcb = to_dev(Kc[:, :s]), to_dev(Kc[:, s:])
    vca, vcb = to_dev(Vc[:, :s]), to_dev(Vc[:, s:])
    del Kc, Vc

    # every buffer allocated before timing
    out = torch.empty_like(q)
    lse = torch.empty((H, N), dtype=torch.float32, device=dev)
    ws_self = torch.empty(sa.sol_attn_workspace_size(N, N, H, d, B, sa.SOL_SPARSE),
                          dtype=torch.uint8, device=dev)
    nq = c["nq"]
    ws_a = torch.empty(max(1, sa.sol_attn_workspace_size(nq, s, H, d, B, sa.SOL_DENSE)),
                       dtype=torch.uint8, device=dev)
    ws_b = torch.empty(max(1, sa.sol_attn_workspace_size(nq, c["nk"] - s, H, d, B, sa.SOL_DENSE)),
                       dtype=torch.uint8, device=dev)
    oa = torch.empty_like(qc)
    ob = torch.empty_like(qc)
    om = torch.empty_like(qc)
    la = torch.empty((H, nq), dtype=torch.float32, device=dev)
    lb = torch.empty_like(la)
    lm = torch.empty_like(la)
    stream = torch.cuda.current_stream()

    def self_attn(beta=args.beta, mode=sa.SOL_SPARSE):
        sa.sol_attn_forward(q, k, v, B=B, beta=beta, mode=mode, workspace=ws_self, out=out,
                            lse=lse)

    def cross_attn():
        sa.sol_attn_forward(qc, kca, vca, mode=sa.SOL_DENSE, workspace=ws_a, out=oa, lse=la)
        sa.sol_attn_forward(qc, kcb, vcb, mode=sa.SOL_DENSE, workspace=ws_b, out=ob, lse=lb)
        sa.attn_lse_merge(oa, la, ob, lb, out=om, lse=lm)

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        self_attn()
        cross_attn()
    torch.cuda.synchronize()

    # timed region: K steps, HIP events on the launch stream around each part
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        self_attn()
        ev[i][1].record(stream)
        cross_attn()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    self_ms = [ev[i][0].elapsed_time(ev[i][1]) for i in range(args.steps)]
    cross_ms = [ev[i][1].elapsed_time(ev[i][2]) for i in range(args.steps)]
    step_ms = wall * 1e3 / args.steps
    log(f"step {step_ms:.3f} ms  self {np.median(self_ms):.3f} ms  cross {np.median(cross_ms):.3f} ms")

    # routing kernels alone (same kernels as inside the call), to split the call;
    # from 128 key blocks on the call computes the statistics in moment form.
    # The tile schedule call runs the call's whole prefix (pool with the
    # forward's forms, statistics, per-tile work and order), so the fused
    # kernel's time is the call's minus the schedule call's.
    nrep = max(3, args.steps)
    e = [torch.cuda.Event(enable_timing=True) for _ in range(4 * nrep)]
    moment = (N + B - 1) // B >= 128
    n_qt = (N + 127) // 128
    ordered = H * n_qt >= ORDER_MIN_TILES and n_qt <= ORDER_MAX_TILES
    mws = torch.empty(H * (2 * 128 * 128 * 2 + 128 * 4 + 8 * (128 * 128 + 2 * 128) * 4),
                      dtype=torch.uint8, device=q.device)
    for i in range(nrep):
        e[4 * i].record(stream)
        kb_, vb_ = sa.sol_attn_pool(k, v, B)
        e[4 * i + 1].record(stream)
        if moment:
            mu, sigma = sa.sol_attn_row_stats_moment(q, kb_, B, N, workspace=mws)
        else:
            mu, sigma = sa.sol_attn_row_stats(q, kb_, B, N)
        e[4 * i + 2].record(stream)
        if ordered:
            sa.sol_attn_tile_schedule(q, k, v, B=B, beta=args.beta, workspace=ws_self)
        e[4 * i + 3].record(stream)
    torch.cuda.synchronize()
    med = lambda a, b: float(np.median([e[4 * i + a].elapsed_time(e[4 * i + b]) for i in range(nrep)]))
    pool_ms, stats_ms = med(0, 1), med(1, 2)
    call_ms = float(np.mean(self_ms))
    if ordered:
        sched_ms = med(2, 3)  # pool + forms + statistics + tile work and order
        order_ms = sched_ms - pool_ms - stats_ms
        fwd_ms = call_ms - sched_ms
    else:
        order_ms = 0.0
        fwd_ms = call_ms - pool_ms - stats_ms  # includes the forms kernel (about 13 us at 4K)

    # achieved density (outside the timed region)
    _, counts = sa.sol_attn_block_mask(q, kb_, mu, sigma, args.beta, B, N, want_mask=False)
    cnt = counts.cpu().numpy().astype(np.int64)
    nb = (N + B - 1) // B
    rho_row = cnt[0] / (H * N * nb)
    rho_tile32 = cnt[1] / (H * ((N + 31) // 32) * nb)
    rho_tile128 = cnt[2] / cnt[3]

    dense_flops = 4.0 * H * N * N * d
    cross_flops = 4.0 * H * nq * c["nk"] * d
    step_flops = dense_flops + cross_flops
    value = step_flops / (step_ms * 1e-3) / 1e12
    call_tflops = dense_flops / (call_ms * 1e-3) / 1e12

    # roofline of the dominant kernel (fused sparse forward): algorithmic flops
    # = 4 d n_j per selected (row, block) pair
    alg_flops = 4.0 * d * B * cnt[0]
    achieved = alg_flops / (fwd_ms * 1e-3) / 1e12
    executed = 4.0 * d * B * 32 * cnt[1] / (fwd_ms * 1e-3) / 1e12
    # HBM bytes per launch of the fused kernel: calibrated rocprofv3
    # FETCH_SIZE / WRITE_SIZE counters of the same kernel source (null once the
    # source has changed since the counters were taken)
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        try:
            tf = json.load(open(TRAFFIC_FILE))
            if tf.get("kernel_hash") == kernel_hash() and abs(tf.get("beta", -1) - args.beta) < 1e-9:
                traffic = tf.get("bytes_per_launch")
        except Exception:
            traffic = None
    roofline = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic,
                "traffic_source": os.path.relpath(TRAFFIC_FILE, ROOT) if traffic else None,
                "work": "4 d B flop per selected (row, block) pair",
                "executed_tile_tflops": executed,
                "executed_tile_frac": executed / PEAK_BF16_TFLOPS,
                "executed_work": "4 d 32 B flop per (32-row tile, block) pair with a selection"}

    # routing kernels against the HBM roof: pool reads K and V once and writes
    # the fp32 means; the moment-form statistics read Q once (plus the pooled
    # keys for the moments) and write mu and sigma
    pool_bytes = 2.0 * H * N * d * 2 + 2.0 * H * nb * d * 4
    stats_bytes = 1.0 * H * N * d * 2 + H * nb * d * 4 + 2.0 * H * N * 4
    hbm = {
        "pool": {"ms": pool_ms, "bytes": pool_bytes, "gbs": pool_bytes / pool_ms / 1e6,
                 "frac": pool_bytes / pool_ms / 1e6 / PEAK_HBM_GBS},
        "row_stats_moment": {"ms": stats_ms, "bytes": stats_bytes,
                             "gbs": stats_bytes / stats_ms / 1e6,
                             "frac": stats_bytes / stats_ms / 1e6 / PEAK_HBM_GBS},
    }

    extras = {}
    if not args.no_extras:
        for beta2 in (1.0,):
            es = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            self_attn(beta2)
            es[0].record(stream)
            for _ in range(3):
                self_attn(beta2)
            es[1].record(stream)
            torch.cuda.synchronize()
            ms = es[0].elapsed_time(es[1]) / 3
            _, c2 = sa.sol_attn_block_mask(q, kb_, mu, sigma, beta2, B, N, want_mask=False)
            c2 = c2.cpu().numpy()
            extras[f"4k_sparse_beta{beta2}"] = {
                "ms_per_call": ms, "dense_equiv_tflops": dense_flops / ms / 1e9,
                "rho_row": c2[0] / (H * N * nb), "rho_tile128": c2[2] / c2[3]}
        es = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        es[0].record(stream)
        for _ in range(2):
            self_attn(float("-inf"), sa.SOL_DENSE)
        es[1].record(stream)
        torch.cuda.synchronize()
        ms = es[0].elapsed_time(es[1]) / 2
        extras["4k_dense"] = {"ms_per_call": ms, "tflops": dense_flops / ms / 1e9,
                              "pct_bf16_peak": 100 * dense_flops / ms / 1e9 / PEAK_BF16_TFLOPS}
        extras["4k_sparse_kv_sharded"] = kv_sharded(sa, torch, q, k, v, B, args.beta, stream,
                                                    dense_flops, call_ms)
        extras["cross_attention_unsplit"] = cross_unsplit(sa, torch, qc, (kca, kcb), (vca, vcb),
                                                          stream, float(np.mean(cross_ms)))
        extras["fp8_projection_4k"] = fp8_projection(sa, torch, N, H * d, q.device, stream)
        log("tiny, stage-1 and stage-2 workloads")
        extras["tiny"] = workload_lines(sa, torch, "tiny", to_dev, stream, reps=20)
        extras["stage1_768x512"] = workload_lines(sa, torch, "stage1", to_dev, stream)
        extras["stage2_1536x1024"] = workload_lines(sa, torch, "stage2", to_dev, stream)
        extras["stage2_per_token_stress"] = workload_lines(sa, torch, "stage2", to_dev, stream,
                                                           per_token=True)
        extras["na3d_decoder_tile_4k"] = na3d_decoder_tile(sa, torch, q.device, stream)

    cpu = None
    if not args.no_cpu:
        log("cpu oracle baseline")
        cpu = cpu_baseline(Q, K, V, B, args.beta, args.cpu_seconds)
        gpu_ms = {"cross_head": float(np.mean(cross_ms)) / H}
        if "tiny" in extras:
            gpu_ms["tiny"] = extras["tiny"]["beta_0.0"]["ms_per_call"]
            gpu_ms["stage1"] = extras["stage1_768x512"]["beta_0.5"]["ms_per_call"]
        log("cpu oracle full calls (tiny, stage-1, one cross-attention head)")
        cpu["full_calls"] = cpu_full_calls(gpu_ms)

    rec = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s (dense-equivalent)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "4k-stage2-sparse-self-attention+audio-video-cross-attention",
            "self": {"heads": H, "tokens": N, "head_dim": d, "block": B, "beta": args.beta,
                     "centres": w.centres, "seed": w.seed},
            "cross": {"heads": H, "queries": nq, "keys": c["nk"], "halves": [s, c["nk"] - s],
                      "seed": c["seed"]},
            "parallelism": "single-gpu",
        },
        "ms_per_call_4k_sparse": call_ms,
        "ms_per_call_4k_sparse_median": float(np.median(self_ms)),
        "ms_per_call_4k_sparse_min": float(np.min(self_ms)),
        "dense_equiv_tflops_4k_sparse": call_tflops,
        "pct_bf16_peak_4k_sparse": 100 * call_tflops / PEAK_BF16_TFLOPS,
        "components_ms": {"pool": pool_ms, "row_stats": stats_ms,
                          "forms_tile_work_and_order": order_ms,
                          "fused_forward": fwd_ms,
                          "cross_attention_halves_plus_merge": float(np.mean(cross_ms))},
        "density": {"rho_row": rho_row, "rho_tile32": rho_tile32, "rho_tile128": rho_tile128},
        "routing_hbm": hbm,
        "cross_attention_hbm": {
            "ms": float(np.mean(cross_ms)), "bytes": 2.0 * H * c["nk"] * d * 2,
            "gbs": 2.0 * H * c["nk"] * d * 2 / float(np.mean(cross_ms)) / 1e6,
            "frac": 2.0 * H * c["nk"] * d * 2 / float(np.mean(cross_ms)) / 1e6 / PEAK_HBM_GBS,
            "work": "two split-KV halves + merge; K and V read once"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extras": extras,
        "kernel_hash": kernel_hash(),
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

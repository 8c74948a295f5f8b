/*
 * solattn.h -- C ABI of the MI355X (gfx950) query-thresholded block-sparse
 * attention library (libsolattn.so).
 *
 * The operation (Sol-Attn style, training-free):
 *   "Accelerating LTX-2.5 with Sol Engine" (NVlabs Sana Sol-Engine/LTX25 page),
 *   section "Stage 2 Optimization -- Core Technology: Sol-Attn":
 *     - each query row i derives a threshold tau_i = mu_i + beta * sigma_i from
 *       the statistics of its block proxy scores (bullet "Query-dependent
 *       thresholding");
 *     - pooled keys are streamed chunk-wise and compared with the threshold
 *       inside the online-softmax pass, with no proxy map stored (bullet
 *       "On-the-fly routing");
 *     - rejected blocks are approximated by a Taylor expansion about the
 *       row-wise mean score (bullet "Proxy-score reuse").
 *   The pages give the Taylor term only in words.  This library fixes it as:
 *   a rejected key block j (n_j valid tokens, mean key kbar_j, mean value
 *   vbar_j) contributes weight w_ij = n_j * e^{mu_i} * (1 + p_ij - mu_i) on
 *   vbar_j to the numerator and w_ij to the denominator, where
 *   p_ij = q_i . kbar_j / sqrt(d) and mu_i, sigma_i are the mean and the
 *   population standard deviation of p_i. over all key blocks.  Selected
 *   blocks (p_ij >= tau_i) are attended exactly.  beta = -inf is plain dense
 *   softmax attention.
 *
 *   "LTX-2.5 at 4K, in half the time" (doubleAI page), section "Attention
 *   across two GPUs": partial answers over disjoint key sets carry their
 *   log-sum-exp and merge exactly (attn_lse_merge); the work of a short query
 *   is split along the keys (done inside sol_attn_forward); a ragged key count
 *   is handled by dropping, never padding, the missing keys.
 *
 * Conventions shared by every entry point:
 *   - Tensors are row-major, contiguous, [H, rows, d]; batch folds into H.
 *     bf16 tensors are passed as uint16_t bit patterns.
 *   - All pointers are device pointers (HIP device memory) unless stated.
 *     The caller owns every buffer.  Inputs are only read; outputs are
 *     written in full.  The library never allocates, frees or synchronises:
 *     all work is enqueued on `stream` (a hipStream_t; NULL = null stream).
 *   - Softmax scale is 1/sqrt(d).  Only d = 128 is supported; B is 64 or 128.
 *   - Return codes: SOL_OK, or a negative SOL_ERR_*.  Arguments are checked
 *     before anything is enqueued: SOL_ERR_INVALID_ARG and SOL_ERR_UNSUPPORTED
 *     mean nothing was launched.  SOL_ERR_HIP reports the failure of one of
 *     the call's own kernel launches (the status that launch returned, never
 *     an earlier error pending on the thread); launches of the same call
 *     that precede it stay enqueued, and the outputs are then undefined.
 *   - Stateless and thread-safe.  Calls on different streams that write
 *     disjoint outputs may overlap.
 *   - Offsets are 64-bit throughout (a 4K sequence of 130,686 tokens times 32
 *     heads times 128 dims exceeds 2^31 bytes).
 */
#ifndef SOLATTN_H
#define SOLATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The library is built with hidden symbols by default; exactly the
 * declarations below are exported. */
#if defined(__GNUC__)
#pragma GCC visibility push(default)
#endif

/* return codes */
#define SOL_OK 0
#define SOL_ERR_INVALID_ARG (-1) /* null pointer, size <= 0, NaN beta, short workspace, misalignment */
#define SOL_ERR_UNSUPPORTED (-2) /* d != 128, B not in {64, 128}, unknown mode */
#define SOL_ERR_HIP (-3)         /* the HIP runtime reported a launch error */
#define SOL_ERR_SCRATCH (-4)     /* sol_attn_forward_noalloc: the call needs more than its scratch */

/* modes of sol_attn_forward */
#define SOL_DENSE 0  /* plain softmax attention; beta and B are ignored */
#define SOL_SPARSE 1 /* thresholded block-sparse attention with the Taylor term */

/*
 * Block mean-pool of keys and values.
 *   Sol-Engine LTX25 page, "Stage 2 Optimization -- Core Technology: Sol-Attn",
 *   bullets "On-the-fly routing" (pooled keys) and "Proxy-score reuse".
 * k, v     [H, N, d] bf16 (read).
 * kbar     [H, nb, d] fp32 (written), nb = ceil(N / B): row j is the mean of
 *          keys jB .. min(N, (j+1)B) - 1 (the last block may hold fewer than B
 *          tokens; only real tokens are averaged).
 * vbar     [H, nb, d] fp32 (written), the same for values.
 * Pointers 16-byte aligned.
 */
int sol_attn_pool(const uint16_t* k, const uint16_t* v, float* kbar, float* vbar,
                  int N, int H, int d, int B, void* stream);

/*
 * Row statistics of the block proxy scores (the first half of the routing).
 *   Sol-Engine LTX25 page, "Stage 2 Optimization -- Core Technology: Sol-Attn",
 *   bullet "Query-dependent thresholding".
 * q        [H, N, d] bf16 query rows (read).
 * kbar     [H, nb, d] fp32 pooled keys of Nk keys, nb = ceil(Nk / B) (read).
 * mu       [H, N] fp32 (written): mean over j of p_ij = q_i . kbar_j / sqrt(d).
 * sigma    [H, N] fp32 (written): population standard deviation of p_i. .
 * The proxy map p is never stored.
 */
int sol_attn_row_stats(const uint16_t* q, const float* kbar, float* mu, float* sigma,
                       int N, int Nk, int H, int d, int B, void* stream);

/*
 * The same statistics in moment form, as sol_attn_forward computes them from
 * 128 key blocks on: p_ij - mu_i = q_i . (kbar_j - mbar) / sqrt(d) is linear
 * in q_i, so mu_i = q_i . mbar / sqrt(d) and sigma_i^2 = q_i^T C q_i / d, with
 * mbar the mean and C the population covariance of the pooled keys of a head.
 * Equal to sol_attn_row_stats up to rounding, at 2 d^2 instead of 2 d nb
 * multiply-adds per row.
 * Arguments as sol_attn_row_stats, plus:
 * workspace  device scratch of at least H * (2 * d * d * 2 + d * 4 +
 *            8 * (d * d + 2 * d) * 4) bytes, 256-byte aligned, caller-owned;
 *            on return it holds C (bf16 hi and lo parts), mbar and the partial
 *            sums of 8 ranges of blocks, in that order.
 * ws_bytes   its size; smaller returns SOL_ERR_INVALID_ARG before any launch.
 */
int sol_attn_row_stats_moment(const uint16_t* q, const float* kbar, float* mu, float* sigma,
                              int N, int Nk, int H, int d, int B, void* workspace,
                              size_t ws_bytes, void* stream);

/*
 * Attention forward.
 *   SOL_SPARSE: Sol-Engine LTX25 page, "Stage 2 Optimization -- Core
 *   Technology: Sol-Attn" (all three bullets), with the Taylor weight above.
 *   SOL_DENSE, or SOL_SPARSE with beta = -inf: plain softmax attention.
 *   beta = +inf selects no block (every block enters through its Taylor term).
 * q        [H, N, d] bf16, N query rows (read).
 * k, v     [H, Nk, d] bf16, Nk key rows (read); Nk = 0 means Nk = N.
 * out      [H, N, d] bf16 (written, round to nearest even).
 * lse      [H, N] fp32 natural log of the full softmax denominator (exact plus
 *          Taylor mass) relative to e^0, or NULL.
 * B        key block size for SOL_SPARSE (64 or 128); ignored by SOL_DENSE.
 * beta     threshold multiplier; NaN is an error.
 * workspace, ws_bytes: device scratch of at least
 *          sol_attn_workspace_size(N, Nk, H, d, B, mode) bytes, 256-byte
 *          aligned (may be NULL when that size is 0).  Its contents on entry
 *          are ignored; on return it holds kbar, vbar, mu, sigma (sparse) and
 *          split partials.  Two calls in flight must not share a workspace.
 * When few query tiles exist (short queries against long keys), the keys are
 * split across workgroups and the partial answers are merged exactly
 * (doubleAI page, "Attention across two GPUs").
 */
int sol_attn_forward(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                     uint16_t* out, float* lse, int N, int H, int d, int B,
                     float beta, int mode, int Nk, void* workspace, size_t ws_bytes,
                     void* stream);

/* Bytes of workspace sol_attn_forward needs for these sizes (0 if none). */
size_t sol_attn_workspace_size(int N, int Nk, int H, int d, int B, int mode);

/*
 * sol_attn_forward without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, checks, kernels and
 * results as sol_attn_forward, minus workspace and ws_bytes: the work space
 * is a 128 MiB array inside the library, one per GPU, held from the library's
 * load until the process ends (it covers the 4K latent workload:
 * sol_attn_workspace_size(130686, 0, 32, 128, 128, SOL_SPARSE) is 106 MiB).
 * The caller still passes q, k, v, out and lse.  No allocation or free is
 * made.  The array of the GPU that runs `stream` is used (on its first use
 * per GPU the library looks its address up once and keeps it).
 * Returns SOL_ERR_SCRATCH, before any launch, when
 * sol_attn_workspace_size(N, Nk, H, d, B, mode) exceeds 128 MiB.
 * All calls on one GPU share its array: two calls that overlap in time on
 * one GPU (different streams, or graph replays in flight) race and give
 * undefined results; calls that follow each other on a stream are safe.  No
 * array contents need clearing: every call writes all it reads.
 */
int sol_attn_forward_noalloc(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                             uint16_t* out, float* lse, int N, int H, int d, int B, float beta,
                             int mode, int Nk, void* stream);

/*
 * Inspection: the order in which sol_attn_forward (SOL_SPARSE) runs the
 * 128-row query tiles of each head.
 *   Sol-Engine LTX25 page, "Stage 2 Optimization -- Core Technology: Sol-Attn",
 *   bullet "Query-dependent thresholding": every row selects its own key
 *   blocks, so the 128-row tiles of a head carry different amounts of work
 *   (the blocks any of their rows selects).
 * The forward call, for a sparse call without a key split and with at least
 * 2048 tiles in all (4 x 2 x 256 CUs) and at most 4096 tiles per head, counts
 * each tile's work and launches each head's tiles in order of decreasing work
 * (ties by tile index); the order decides only when a tile runs, never its
 * result.  This entry point runs the same steps (pool, row statistics, work
 * count, ranking) for any such call size and returns their results:
 * work     [H, ceil(N/128)] int32 (written): per tile, the key blocks one of
 *          its rows selects -- by the forward predicate on proxy scores from
 *          the bf16 high part of the pooled keys, so a pair within about
 *          2^-9 of its row's threshold scale may count differently from the
 *          forward kernel's decision.
 * order    [H * ceil(N/128)] int32 (written): order[h * n + r] = h * n + t
 *          for the tile t of head h that runs r-th (n = ceil(N/128)).
 * q, k, v, N, H, d, B, beta, Nk as sol_attn_forward (SOL_SPARSE); beta = -inf
 * is SOL_ERR_INVALID_ARG (nothing to count), more than 4096 tiles per head
 * SOL_ERR_UNSUPPORTED.
 * workspace, ws_bytes: at least sol_attn_workspace_size(N, Nk, H, d, B,
 *          SOL_SPARSE) bytes, 256-byte aligned.
 * work and order 4-byte aligned, q, k, v 16-byte aligned (SOL_ERR_INVALID_ARG
 * otherwise).
 */
int sol_attn_tile_schedule(const uint16_t* q, const uint16_t* k, const uint16_t* v, int* work,
                           int* order, int N, int H, int d, int B, float beta, int Nk,
                           void* workspace, size_t ws_bytes, void* stream);

/*
 * Exact merge of two partial answers over disjoint key sets.
 *   doubleAI page, "Attention across two GPUs": each partial carries its
 *   running maximum and sum of exponentials (here as lse) and merges exactly.
 * out_a, out_b [H, N, d] bf16 and lse_a, lse_b [H, N] fp32 (read).
 * out [H, N, d] bf16 and lse [H, N] fp32 (written):
 *   lse = log(e^lse_a + e^lse_b), out = e^(lse_a-lse) out_a + e^(lse_b-lse) out_b.
 * Both lse = -inf gives out = 0, lse = -inf.  out may alias out_a (or out_b)
 * and lse may alias lse_a (or lse_b).
 */
int attn_lse_merge(const uint16_t* out_a, const float* lse_a, const uint16_t* out_b,
                   const float* lse_b, uint16_t* out, float* lse, int N, int H, int d,
                   void* stream);

/*
 * Key-sharded Sol-Attn, one rank's share: the partial answer of all N query
 * rows over this rank's key blocks.
 *   doubleAI page, "Attention across two GPUs": the keys are split along the
 *   sequence, each GPU attends to its part, and the partial answers (each
 *   with its running maximum and sum of exponentials) merge exactly.
 *   Sol-Engine LTX25 page, "Stage 2 Optimization -- Core Technology:
 *   Sol-Attn": a row's threshold comes from the proxy statistics of the
 *   whole sequence, so every share uses the same mu_i, sigma_i; the exact and
 *   the Taylor parts are sums over key blocks, so the shares add up exactly.
 * q        [H, N, d] bf16: every query row (read).
 * k, v     [H, Nk, d] bf16 (read): this rank's keys, whole key blocks of B of
 *          the full sequence starting at a block boundary (only the last rank's
 *          share may end in a ragged block).
 * kbar_all [H, nb_all, d] fp32 (read): the pooled keys of every block of the
 *          full sequence (each rank's sol_attn_pool output, gathered), used for
 *          mu_i and sigma_i.  Ignored (may be NULL) when beta = -inf.
 * part_o   [H, N, d] fp32 (written): the share's numerator relative to 2^m.
 * part_ml  [H, N, 2] fp32 (written): m (log2 units) and the share's signed
 *          denominator relative to 2^m (a share of rejected blocks alone can
 *          have a negative one; the merge stays exact).
 * beta     as sol_attn_forward (SOL_SPARSE); -inf gives the dense partial.
 * workspace, ws_bytes: at least sol_attn_shard_workspace_size(...) bytes,
 *          256-byte aligned (may be NULL when that size is 0).
 * The share runs without a further key split inside the call.  16-byte
 * aligned pointers (part_ml: 8).  Merge shares with sol_attn_combine_partials.
 */
int sol_attn_forward_shard(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                           const float* kbar_all, float* part_o, float* part_ml, int N,
                           int Nk, int nb_all, int H, int d, int B, float beta,
                           void* workspace, size_t ws_bytes, void* stream);

/* Bytes of workspace sol_attn_forward_shard needs (0 if none). */
size_t sol_attn_shard_workspace_size(int N, int Nk, int nb_all, int H, int d, int B,
                                     float beta);

/*
 * Exact merge of S partial answers in (numerator, m, denominator) form.
 *   doubleAI page, "Attention across two GPUs".
 * part_o   [S, H, N, d] fp32 and part_ml [S, H, N, 2] fp32 (read): share s at
 *          index s (e.g. gathered from S ranks' sol_attn_forward_shard).
 * out      [H, N, d] bf16 (written): sum_s 2^(m_s-M) o_s / sum_s 2^(m_s-M) l_s.
 * lse      [H, N] fp32 natural log of the merged denominator, or NULL.
 */
int sol_attn_combine_partials(const float* part_o, const float* part_ml, int S, uint16_t* out,
                              float* lse, int N, int H, int d, void* stream);

/* Static description of a return code (never NULL). */
const char* sol_attn_error_string(int code);

/*
 * Inspection: proxy scores of a row range, p_ij = q_i . kbar_j / sqrt(d),
 * computed by the same device code the forward kernel uses for routing.
 *   Sol-Engine LTX25 page, "Stage 2 Optimization -- Core Technology: Sol-Attn".
 * p        [H, nrows, nb] fp32 (written) for rows row0 .. row0 + nrows - 1.
 */
int sol_attn_proxy_scores(const uint16_t* q, const float* kbar, float* p, int row0,
                          int nrows, int N, int Nk, int H, int d, int B, void* stream);

/*
 * Inspection: the block selection the forward kernel makes, for rows
 * row0 .. row0 + nrows - 1 (row0 a multiple of 128), and density counts.
 *   Sol-Engine LTX25 page, "Stage 2 Optimization -- Core Technology: Sol-Attn",
 *   bullet "Query-dependent thresholding" (p_ij >= mu_i + beta sigma_i).
 * mask     [H, nrows, nb] uint8 (written, 1 = attended exactly), or NULL.
 * counts   int64[4] (written): selected (row, block) pairs; (32-row tile, block)
 *          pairs with any selected row; (128-row tile, block) pairs with any
 *          selected row; number of (128-row tile, block) pairs in the range.
 * mu, sigma from sol_attn_row_stats.  beta as in sol_attn_forward.
 */
int sol_attn_block_mask(const uint16_t* q, const float* kbar, const float* mu,
                        const float* sigma, float beta, int row0, int nrows, int N,
                        int Nk, int H, int d, int B, uint8_t* mask, int64_t* counts,
                        void* stream);

/*
 * FP8 projection GEMM around attention: weights stay in FP8, activations are
 * converted to FP8 with one scale per row, products accumulate in FP32.
 *   [DAI] "LTX-2.5 at 4K, in half the time" (doubleAI), section "Thinner seams".
 * FP8 is E4M3 in its finite-only form (bias 7, largest finite value 448).
 *
 * fp8_quantize_rows: per-row quantisation of a bf16 matrix.
 * x      [M, K] bf16 row-major (read), finite values; 16-byte aligned.
 * q      [M, K] E4M3 codes (written): q_ik = RNE(x_ik * (448 / amax_i)), the
 *        product formed in fp32 and clamped to +-448; 8-byte aligned.
 * scale  [M] fp32 (written): amax_i / 448 (0 for an all-zero row, whose codes
 *        are 0).
 * K must be a multiple of 8 (SOL_ERR_UNSUPPORTED otherwise).
 */
int fp8_quantize_rows(const uint16_t* x, uint8_t* q, float* scale, int64_t M, int K,
                      void* stream);

/*
 * fp8_gemm_rowscale: y[m, n] = sa[m] * sw[n] * sum_k dec(a[m, k]) * dec(w[n, k]),
 * accumulated in fp32 on the FP8 matrix cores, written as bf16 (round to
 * nearest even).
 * a    [M, K] E4M3 activations (read), sa [M] fp32 their row scales.
 * w    [N, K] E4M3 weights, one row per output channel (read), sw [N] fp32.
 * y    [M, N] bf16 (written).
 * K and N must be multiples of 128 (SOL_ERR_UNSUPPORTED otherwise); a, w, sw
 * and y 16-byte aligned.  No workspace; nothing is allocated.
 */
int fp8_gemm_rowscale(const uint8_t* a, const float* sa, const uint8_t* w, const float* sw,
                      uint16_t* y, int M, int N, int K, void* stream);

/*
 * 3D neighbourhood attention over a video token grid (the diffusion video
 * decoder's attention).
 *   [DAI] "LTX-2.5 at 4K, in half the time" (doubleAI), section "Inside the
 *   decoder"; the na3d backends named by the LTX-2 pipelines optimization guide.
 * The query at (t, y, x) attends to the kt x ky x kx keys of the window centred
 * on it and shifted inward at the borders (start clamp(p - k/2, 0, L - k) per
 * axis), softmax with scale 1/sqrt(d).
 * q, k, v  [H, T*Y*X, d] bf16 (read), tokens frame-major then row-major.
 * out      [H, T*Y*X, d] bf16 (written).  lse [H, T*Y*X] fp32 (may be NULL).
 * kt, ky, kx odd and at most T, Y, X (SOL_ERR_INVALID_ARG otherwise);
 * d = 128 and kx <= 25 (SOL_ERR_UNSUPPORTED otherwise).  16-byte alignment.
 */
int na3d_forward(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* out,
                 float* lse, int T, int Y, int X, int H, int d, int kt, int ky, int kx,
                 void* stream);

#if defined(__GNUC__)
#pragma GCC visibility pop
#endif

#ifdef __cplusplus
}
#endif

#endif /* SOLATTN_H */

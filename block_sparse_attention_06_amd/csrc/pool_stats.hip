// Routing kernels: block mean-pool, proxy-score row statistics, the launch
// order of a sparse call's query tiles (per-tile work count and per-head
// ranking), and the two inspection kernels (proxy scores of a row range,
// block selection mask).
//
// Sol-Engine LTX25 page, "Stage 2 Optimization -- Core Technology: Sol-Attn":
// pooled keys give per-row block proxy scores whose mean and spread set the
// row's threshold.  All of this is HBM- or L2-bound; nothing here stores the
// proxy map of a full sequence.
#include "device.hpp"
#include "launch.hpp"

namespace solattn {

// ---------------------------------------------------------------------------
// Block mean-pool.  One workgroup per (key block j, head h, tensor K|V).
// 256 threads = 16 row groups x 16 column chunks of 8 bf16 (16 B): every load
// instruction of a wave reads 4 whole 256-byte rows (coalesced, non-temporal:
// the keys and values are read once here), and each thread keeps all its row
// loads in flight before summing.
// ---------------------------------------------------------------------------
template <int B>
__global__ __launch_bounds__(256) void pool_kernel(PoolArgs a) {
  __shared__ float part[16][kHeadDim + 4];
  const int j = blockIdx.x, h = blockIdx.y, which = blockIdx.z;
  const int tid = threadIdx.x, chunk = tid & 15, rg = tid >> 4;
  const uint16_t* src = (which ? a.v : a.k) + ((int64_t)h * a.N + (int64_t)j * B) * kHeadDim;
  const int n = min(B, a.N - j * B);
  constexpr int R = B / 16;
  u32x4 x[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    int t = rg + 16 * r;
    x[r] = t < n ? gload_nt<u32x4>(src + (int64_t)t * kHeadDim + chunk * 8) : u32x4{0u, 0u, 0u, 0u};
  }
  float acc[8] = {};
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += __uint_as_float(x[r][e] << 16);
      acc[2 * e + 1] += __uint_as_float(x[r][e] & 0xffff0000u);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[rg][chunk * 8 + e] = acc[e];
  __syncthreads();
  if (tid < kHeadDim) {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += part[r][tid];
    float* dst = which ? a.vbar : a.kbar;
    dst[((int64_t)h * a.nb + j) * kHeadDim + tid] = s / (float)n;
  }
}

// ---------------------------------------------------------------------------
// Routing forms of the pooled blocks for the fused forward kernel.  One
// workgroup per (16 consecutive blocks, head), blocks up to nb_pad:
//  - khi / klo: the bf16 hi + lo parts of the pooled keys, rows past the last
//    block zero (whole 16-byte stores);
//  - vsumT: the value block sums n_j * vbar_j in bf16, transposed to
//    [dim][block] with the blocks of each group of 16 permuted for the Taylor
//    MFMA operand; staged in LDS so that each dimension's 32 bytes go out as
//    two 16-byte stores.
// The pool kernel itself only writes the fp32 means, coalesced.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void forms_kernel(PoolArgs a) {
  __shared__ __attribute__((aligned(16))) u16 vs[kHeadDim][16];
  const int h = blockIdx.y, tid = threadIdx.x;
  const int j0 = blockIdx.x * 16, jj = tid >> 4, c = (tid & 15) * 8, j = j0 + jj;
  f32x4 k0 = {0.f, 0.f, 0.f, 0.f}, k1 = k0, v0 = k0, v1 = k0;
  float n = 0.f;
  if (j < a.nb) {
    const float* kb = a.kbar + ((int64_t)h * a.nb + j) * kHeadDim + c;
    const float* vb = a.vbar + ((int64_t)h * a.nb + j) * kHeadDim + c;
    k0 = *reinterpret_cast<const f32x4*>(kb);
    k1 = *reinterpret_cast<const f32x4*>(kb + 4);
    v0 = *reinterpret_cast<const f32x4*>(vb);
    v1 = *reinterpret_cast<const f32x4*>(vb + 4);
    n = (float)min(a.B, a.N - j * a.B);  // valid keys of the block
  }
  bf16x8 hi, lo;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    __bf16 hh, ll;
    split_bf16(k0[e], hh, ll);
    hi[e] = hh;
    lo[e] = ll;
    split_bf16(k1[e], hh, ll);
    hi[e + 4] = hh;
    lo[e + 4] = ll;
  }
  const int64_t ko = ((int64_t)h * a.nb_pad + j) * kHeadDim + c;
  *reinterpret_cast<bf16x8*>(a.khi + ko) = hi;
  *reinterpret_cast<bf16x8*>(a.klo + ko) = lo;
  const int pj = perm16(jj);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    vs[c + e][pj] = f32_to_bf16_bits(v0[e] * n);
    vs[c + 4 + e][pj] = f32_to_bf16_bits(v1[e] * n);
  }
  __syncthreads();
  const int dim = tid >> 1, half = tid & 1;
  *reinterpret_cast<u32x4*>(a.vsumT + ((int64_t)h * kHeadDim + dim) * a.nb_pad + j0 + half * 8) =
      *reinterpret_cast<const u32x4*>(&vs[dim][half * 8]);
}

hipError_t launch_pool(const PoolArgs& a, hipStream_t s) {
  dim3 grid(a.nb, a.H, 2);
  const hipError_t e = a.B == 64 ? launch_kernel(pool_kernel<64>, grid, dim3(256), s, a)
                                 : launch_kernel(pool_kernel<128>, grid, dim3(256), s, a);
  if (e != hipSuccess) return e;
  // the forward pass's forms (khi, klo and vsumT are set together)
  if (a.khi) return launch_kernel(forms_kernel, dim3(a.nb_pad / 16, a.H), dim3(256), s, a);
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// Row statistics mu_i, sigma_i of p_i. over all key blocks.  One wave per 32
// query rows, four waves per workgroup.  Each chunk of 32 pooled keys is split
// into bf16 hi / lo parts once per workgroup and staged in LDS (16-byte chunk
// c of row r at c ^ (r % 16)), then every wave runs the proxy MFMA sequence on
// it.  Sums are shifted by the row's first proxy p_i0 so the variance has no
// cancellation, then reduced over the two lane halves.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void stats_kernel(StatsArgs a) {
  __shared__ __attribute__((aligned(16))) u16 khi[kChunk * kHeadDim];
  __shared__ __attribute__((aligned(16))) u16 klo[kChunk * kHeadDim];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5;
  const int h = blockIdx.y;
  const int row = blockIdx.x * kQTile + wave * 32 + (lane & 31);
  const bool valid = row < a.N;
  QFrag qf;
  load_qfrag(qf, a.q + (int64_t)h * a.N * kHeadDim, row, valid, g);
  const float* kb = a.kbar + (int64_t)h * a.nb * kHeadDim;
  float shift = 0.f, s1 = 0.f, s2 = 0.f;
  for (int b0 = 0; b0 < a.nb; b0 += kChunk) {
    __syncthreads();
    // 32 rows x 16 chunks of 8 values: two chunks per thread
#pragma unroll
    for (int rep = 0; rep < 2; ++rep) {
      const int idx = tid + 256 * rep, r = idx >> 4, c = idx & 15;
      const int blk = min(b0 + r, a.nb - 1);
      const f32x4* src = reinterpret_cast<const f32x4*>(kb + (int64_t)blk * kHeadDim + c * 8);
      const f32x4 x0 = src[0], x1 = src[1];
      bf16x8 hi, lo;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        __bf16 hh, ll;
        split_bf16(x0[e], hh, ll);
        hi[e] = hh;
        lo[e] = ll;
        split_bf16(x1[e], hh, ll);
        hi[e + 4] = hh;
        lo[e + 4] = ll;
      }
      const int off = r * kHeadDim + ((c ^ (r & 15)) << 3);
      *reinterpret_cast<bf16x8*>(&khi[off]) = hi;
      *reinterpret_cast<bf16x8*>(&klo[off]) = lo;
    }
    __syncthreads();
    const int r = lane & 31;
    const f32x16 p = proxy_tile(qf, [&](int ks, bf16x8& hi, bf16x8& lo) __attribute__((always_inline)) {
      const int off = r * kHeadDim + (((ks * 2 + g) ^ (r & 15)) << 3);
      hi = *reinterpret_cast<const bf16x8*>(&khi[off]);
      lo = *reinterpret_cast<const bf16x8*>(&klo[off]);
    });
    if (b0 == 0) shift = __shfl(p[0], lane & 31);  // block 0 sits in element 0 of lane half 0
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (b0 + acc_row(i, g) < a.nb) {
        const float x = p[i] - shift;
        s1 += x;
        s2 = __builtin_fmaf(x, x, s2);
      }
    }
  }
  s1 += __shfl_xor(s1, 32);
  s2 += __shfl_xor(s2, 32);
  if (g == 0 && valid) {
    const float inv = 1.f / (float)a.nb;
    const float md = s1 * inv;
    const float var = __builtin_fmaf(-md, md, s2 * inv);
    a.mu[(int64_t)h * a.N + row] = shift + md;
    a.sigma[(int64_t)h * a.N + row] = sqrtf(fmaxf(var, 0.f));
  }
}

hipError_t launch_stats(const StatsArgs& a, hipStream_t s) {
  dim3 grid((a.N + kQTile - 1) / kQTile, a.H);
  return launch_kernel(stats_kernel, grid, dim3(256), s, a);
}

// ---------------------------------------------------------------------------
// Row statistics in moment form.  p_ij - mu_i = s q_i . (kbar_j - mbar) is
// linear in q_i, so over the blocks
//   mu_i = s q_i . mbar,   sigma_i^2 = s^2 q_i^T C q_i,
// with mbar the mean of the pooled keys and C their population covariance.
// Same quantities as stats_kernel up to
// rounding, at 2 d^2 instead of 2 d nb multiply-adds per row.
//
// Moments of the pooled keys, in two kernels.  32 keys at a time are staged
// in LDS, shifted by the head's first pooled key (so the second moments carry
// no large common offset: the shift-then-correct form keeps the cancellation
// to the keys' own spread), while the next 32 are already being loaded; each
// thread accumulates 8 entries of the shifted second moment plus the shifted
// sums of its row and columns, all in fp32.
// ---------------------------------------------------------------------------

// Stored position, within its 32-row tile, of row `off` of C.  The MFMA
// accumulator element e of lane half g sits in row 8(e/4) + 4g + e%4 of the
// tile; storing C row 16(b/2) + 8g + 4(b%2) + i (b = e/4, i = e%4) there makes
// element e of lane half g the query dimension that element e % 8 of query
// fragment k-step 2 tile + e / 8 holds in that lane half.
__device__ __forceinline__ int c_row_pos(int off) {
  return 8 * (2 * (off >> 4) + ((off >> 2) & 1)) + 4 * ((off >> 3) & 1) + (off & 3);
}

// moments_part_kernel: workgroup (32 rows of C, block range s, head); the
// pooled keys are split into kMomentSplits contiguous ranges so that no
// workgroup walks all of them.  Wave w owns column block w (32 columns) and
// works only at or right of the diagonal block: the blocks below it are not
// part of the stored form of C.  A lane keeps a 4 x 4 tile and reads one
// 16-byte row operand and one column operand per pooled key.  Each workgroup
// writes its shifted partial sums (second moment over its blocks, sums of its
// 32 rows); moments_final_kernel adds the ranges.  The row sums double as the
// column sums (the same vector of shifted pooled keys summed).
__global__ __launch_bounds__(256) void moments_part_kernel(MomentArgs a) {
  __shared__ __attribute__((aligned(16))) float kc[kChunk][kHeadDim + 4];
  __shared__ __attribute__((aligned(16))) float k0s[kHeadDim];
  const int rb = blockIdx.x, sp = blockIdx.y, h = blockIdx.z, tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const float* kb = a.kbar + (int64_t)h * a.nb * kHeadDim;
  if (tid < kHeadDim) k0s[tid] = kb[tid];
  const int per = (a.nb + kMomentSplits - 1) / kMomentSplits;
  const int jb = min(a.nb, sp * per), je = min(a.nb, jb + per);
  constexpr int kPer = kChunk * kHeadDim / 4 / 256;  // staged 16-byte values per thread
  f32x4 nxt[kPer];
  auto load = [&](int j0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = tid + 256 * i, j = j0 + (e >> 5);
      nxt[i] = j < je ? *reinterpret_cast<const f32x4*>(kb + (int64_t)j * kHeadDim + (e & 31) * 4)
                      : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  load(jb);
  const bool active = wave >= rb;  // wave-uniform
  const int r0 = rb * 32 + (lane >> 3) * 4, c0 = wave * 32 + (lane & 7) * 4;
  float acc[4][4] = {};
  float sr[4] = {0.f, 0.f, 0.f, 0.f};
  for (int j0 = jb; j0 < je; j0 += kChunk) {
    __syncthreads();  // the previous chunk has been consumed (and k0s is visible)
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = tid + 256 * i, jj = e >> 5, cc = (e & 31) * 4;
      const f32x4 k0 = *reinterpret_cast<const f32x4*>(&k0s[cc]);
      const f32x4 x = j0 + jj < je ? nxt[i] - k0 : f32x4{0.f, 0.f, 0.f, 0.f};
      *reinterpret_cast<f32x4*>(&kc[jj][cc]) = x;
    }
    __syncthreads();
    if (j0 + kChunk < je) load(j0 + kChunk);
    if (active) {
      const int nj = min(kChunk, je - j0);
      for (int jj = 0; jj < nj; ++jj) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(&kc[jj][r0]);
        const f32x4 y = *reinterpret_cast<const f32x4*>(&kc[jj][c0]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sr[i] += x[i];
#pragma unroll
          for (int k = 0; k < 4; ++k) acc[i][k] = __builtin_fmaf(x[i], y[k], acc[i][k]);
        }
      }
    }
  }
  float* part = a.part + ((int64_t)h * kMomentSplits + sp) * kMomentPartFloats;
  if (active) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<f32x4*>(part + (r0 + i) * kHeadDim + c0) = f32x4{acc[i][0], acc[i][1], acc[i][2], acc[i][3]};
  }
  if (wave == 3 && (lane & 7) == 0) {  // wave 3 is active for every row block
#pragma unroll
    for (int i = 0; i < 4; ++i) part[kHeadDim * kHeadDim + r0 + i] = sr[i];
  }
}

// moments_final_kernel: workgroup (16 rows of C, head).  Adds the ranges'
// partial sums, then C = S2 / nb - (S1_r / nb)(S1_c / nb), mbar = k0 + S1 / nb.
// C is written as bf16 hi + lo parts (~16 significant bits) in its stored
// block-triangular form, rows permuted (c_row_pos) so that
// stats_moment_kernel's accumulator elements line up with its query fragment.
__global__ __launch_bounds__(256) void moments_final_kernel(MomentArgs a) {
  const int rb = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int r = rb * 16 + (tid >> 4), c0 = (tid & 15) * 8;
  // Stored form: the 32 x 32 blocks of C above the diagonal doubled, those
  // below it zero -- the same quadratic form q^T C q (C is symmetric), with
  // 10 of the 16 blocks left to multiply.  Doubling is exact in both parts.
  const int rbk = r >> 5, cbk = c0 >> 5;
  const bool used = cbk >= rbk;  // blocks below the diagonal have no partial sums
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float sc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float sr = 0.f;
  for (int sp = 0; sp < kMomentSplits; ++sp) {
    const float* part = a.part + ((int64_t)h * kMomentSplits + sp) * kMomentPartFloats;
    const float* sums = part + kHeadDim * kHeadDim;  // row sums (= column sums)
    const f32x4 s0 = *reinterpret_cast<const f32x4*>(sums + c0);
    const f32x4 s1 = *reinterpret_cast<const f32x4*>(sums + c0 + 4);
    sr += sums[r];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      sc[k] += s0[k];
      sc[k + 4] += s1[k];
    }
    if (used) {
      const f32x4 x0 = *reinterpret_cast<const f32x4*>(part + r * kHeadDim + c0);
      const f32x4 x1 = *reinterpret_cast<const f32x4*>(part + r * kHeadDim + c0 + 4);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        acc[k] += x0[k];
        acc[k + 4] += x1[k];
      }
    }
  }
  const float inv_nb = 1.f / (float)a.nb;
  const float mr = sr * inv_nb;
  const float wblk = cbk > rbk ? 2.f : (cbk == rbk ? 1.f : 0.f);
  bf16x8 hi, lo;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    __bf16 hh = (__bf16)0.f, ll = (__bf16)0.f;
    if (used) split_bf16(wblk * __builtin_fmaf(-mr, sc[k] * inv_nb, acc[k] * inv_nb), hh, ll);
    hi[k] = hh;
    lo[k] = ll;
  }
  const int64_t pos = ((int64_t)h * kHeadDim + (r & ~31) + c_row_pos(r & 31)) * kHeadDim + c0;
  *reinterpret_cast<bf16x8*>(a.chi + pos) = hi;
  *reinterpret_cast<bf16x8*>(a.clo + pos) = lo;
  if (rb == 0 && (tid >> 4) == 0) {
    const float* kb = a.kbar + (int64_t)h * a.nb * kHeadDim;
#pragma unroll
    for (int k = 0; k < 8; ++k) a.mbar[(int64_t)h * kHeadDim + c0 + k] = kb[c0 + k] + sc[k] * inv_nb;
  }
}

hipError_t launch_moments(const MomentArgs& a, hipStream_t s) {
  const hipError_t e =
      launch_kernel(moments_part_kernel, dim3(kHeadDim / 32, kMomentSplits, a.H), dim3(256), s, a);
  if (e != hipSuccess) return e;
  return launch_kernel(moments_final_kernel, dim3(kHeadDim / 16, a.H), dim3(256), s, a);
}

// stats_moment_kernel: one wave per 32 query rows, four per 128-row tile, and
// a contiguous range of tiles per workgroup.  Y^T = C Q^T runs on MFMA over
// the stored block-triangular C: row tile ct takes the k-steps of column
// blocks ct .. 3 only (20 of 32 k-steps, x (hi, lo)); each lane dots the
// accumulator elements of a row tile with the matching query values, which it
// already holds as MFMA operands, and adds the partner lane's half.  A wave
// takes two query tiles per pass, so each C operand read from LDS feeds two
// products.
//
// The grid is fixed at about three workgroups per CU (kMomentWGs over the
// heads): workgroup x of head h takes the contiguous tile range
// [x nt / G, (x + 1) nt / G) of that head, so C is staged once per workgroup
// and no last round of workgroups runs the chip part-empty.
//
// Only the used blocks of C are staged, once per workgroup: row R of tile ct
// keeps 16-byte chunks 4 ct .. 15, at positions 0 .. 15 - 4 ct of a row of
// kCW[ct] chunks (an odd count, so that 8 consecutive rows start on different
// banks: conflict-free operand reads).  45 KiB per workgroup; three
// workgroups per CU hide the query loads (there is no register prefetch).
constexpr int kMomentWGs = 3 * 256;  // resident workgroups: three per CU
constexpr int kCW0 = 17, kCW1 = 13, kCW2 = 9, kCW3 = 5;   // padded row widths (chunks)
constexpr int kCBase1 = 32 * kCW0, kCBase2 = kCBase1 + 32 * kCW1, kCBase3 = kCBase2 + 32 * kCW2;
constexpr int kCChunks = kCBase3 + 32 * kCW3;             // 1408 chunks per part

__device__ __forceinline__ int c_width(int ct) { return ct == 0 ? kCW0 : ct == 1 ? kCW1 : ct == 2 ? kCW2 : kCW3; }
__device__ __forceinline__ int c_base(int ct) { return ct == 0 ? 0 : ct == 1 ? kCBase1 : ct == 2 ? kCBase2 : kCBase3; }

__global__ __launch_bounds__(256, 3) void stats_moment_kernel(StatsMomentArgs a) {
  __shared__ __attribute__((aligned(16))) u16 chs[kCChunks * 8];
  __shared__ __attribute__((aligned(16))) u16 cls[kCChunks * 8];
  __shared__ float mb[kHeadDim];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5;
  const int h = blockIdx.y;
  const u16* ch = a.chi + (int64_t)h * kHeadDim * kHeadDim;
  const u16* cl = a.clo + (int64_t)h * kHeadDim * kHeadDim;
  // The 1280 used 16-byte chunks of each part (row tile ct keeps chunks
  // 4 ct .. 15 of its 32 rows: 512, 384, 256, 128 chunks), five per thread,
  // all ten loads issued before the first store.
  u32x4 xh[5], xl[5];
  int soff[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const int e = tid + 256 * i;
    const int ct = (e >= 512) + (e >= 896) + (e >= 1152);
    const int first = ct == 0 ? 0 : ct == 1 ? 512 : ct == 2 ? 896 : 1152;
    const int w = 16 - 4 * ct, le = e - first;
    const int rl = le / w, cu = le - rl * w;
    const int src = (32 * ct + rl) * kHeadDim + (4 * ct + cu) * 8;
    xh[i] = gload<u32x4>(ch + src);
    xl[i] = gload<u32x4>(cl + src);
    soff[i] = (c_base(ct) + rl * c_width(ct) + cu) * 8;
  }
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    *reinterpret_cast<u32x4*>(&chs[soff[i]]) = xh[i];
    *reinterpret_cast<u32x4*>(&cls[soff[i]]) = xl[i];
  }
  if (tid < kHeadDim) mb[tid] = a.mbar[(int64_t)h * kHeadDim + tid];
  const u16* qh = a.q + (int64_t)h * a.N * kHeadDim;
  const int nt = (a.N + kQTile - 1) / kQTile;
  const int t_begin = (int)((int64_t)blockIdx.x * nt / gridDim.x);
  const int t_end = (int)((int64_t)(blockIdx.x + 1) * nt / gridDim.x);
  __syncthreads();
  const int r = lane & 31;
  const float scale = 0.08838834764831845f;  // 1/sqrt(128)
  for (int t = t_begin; t < t_end; t += 2) {
    const int rowa = t * kQTile + wave * 32 + r, rowb = rowa + kQTile;
    const bool va = rowa < a.N, vb = t + 1 < t_end && rowb < a.N;
    QFrag qa, qb;
    load_qfrag(qa, qh, rowa, va, g);
    load_qfrag(qb, qh, rowb, vb, g);
    float s2a = 0.f, s2b = 0.f, s1a = 0.f, s1b = 0.f;
    // an opaque zero: keeps the C operand reads inside the loop (hoisted, the
    // 40 operands of a pass would not fit the register budget)
    int cz = 0;
    asm volatile("" : "+v"(cz));
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      f32x16 ya = {}, yb = {};
      const int rbase = (c_base(ct) + r * c_width(ct) - 4 * ct) * 8 + cz;
#pragma unroll
      for (int ks = 2 * ct; ks < 8; ++ks) {
        const int off = rbase + (ks * 2 + g) * 8;
        const bf16x8 hi = *reinterpret_cast<const bf16x8*>(&chs[off]);
        const bf16x8 lo = *reinterpret_cast<const bf16x8*>(&cls[off]);
        ya = mfma32(hi, qa.k[ks], ya);
        yb = mfma32(hi, qb.k[ks], yb);
        ya = mfma32(lo, qa.k[ks], ya);
        yb = mfma32(lo, qb.k[ks], yb);
      }
      // element e pairs with query dimension 16 (2 ct + e / 8) + 8 g + e % 8;
      // the same values give this tile's part of q . mbar
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int ks = 2 * ct + (e >> 3), k = e & 7;
        const float m = mb[16 * ks + 8 * g + k + cz];
        const float xa = (float)qa.k[ks][k], xb = (float)qb.k[ks][k];
        s2a = __builtin_fmaf(ya[e], xa, s2a);
        s2b = __builtin_fmaf(yb[e], xb, s2b);
        s1a = __builtin_fmaf(xa, m, s1a);
        s1b = __builtin_fmaf(xb, m, s1b);
      }
    }
    s1a += __shfl_xor(s1a, 32);
    s2a += __shfl_xor(s2a, 32);
    s1b += __shfl_xor(s1b, 32);
    s2b += __shfl_xor(s2b, 32);
    if (g == 0 && va) {
      a.mu[(int64_t)h * a.N + rowa] = s1a * scale;
      a.sigma[(int64_t)h * a.N + rowa] = sqrtf(fmaxf(s2a, 0.f)) * scale;
    }
    if (g == 0 && vb) {
      a.mu[(int64_t)h * a.N + rowb] = s1b * scale;
      a.sigma[(int64_t)h * a.N + rowb] = sqrtf(fmaxf(s2b, 0.f)) * scale;
    }
  }
}

hipError_t launch_stats_moment(const StatsMomentArgs& a, hipStream_t s) {
  // workgroups per head: kMomentWGs shared over the heads, at most one per
  // two tiles and at least one
  const int nt = (a.N + kQTile - 1) / kQTile;
  const int per_head = std::max(1, std::min((nt + 1) / 2, kMomentWGs / std::max(1, a.H)));
  dim3 grid(per_head, a.H);
  return launch_kernel(stats_moment_kernel, grid, dim3(256), s, a);
}

// ---------------------------------------------------------------------------
// Order of the query tiles of a sparse call.
//
// The fused kernel loads, for each 128-row tile, every key block one of its
// rows selects, and the two workgroups of each CU stream those blocks through
// the L2 of their XCD.  Workgroups that run at the same time on one XCD share
// those lines only while their key sweeps stay close, which holds when their
// tiles carry about the same work.  So each tile's work -- the number of
// blocks any of its rows selects, by the forward kernel's predicate on proxy
// scores from the high part of the pooled keys -- is counted first, and each
// head's tiles are then launched in order of decreasing work (ties by tile
// index).  The order changes only when a tile runs, never what it computes.
//
// tile_work_kernel: one workgroup per (two 128-row tiles, head), 8 waves of
// 32 rows (waves 0-3 the first tile, 4-7 the second).  The proxy scores use
// the bf16 high part of the pooled keys only: the count ranks tiles, and a
// decision can differ from the forward kernel's only where a proxy lies
// within about 2^-9 of the row's threshold scale.  Each chunk of 32 pooled
// keys (8 KiB) is staged once per workgroup by direct global->LDS loads, one
// instruction per wave, in a ring of three stages filled two chunks ahead;
// chunk c of block row r sits at slot c ^ (r % 16), so the operand reads of
// 16 consecutive rows at one chunk are conflict-free.  One barrier per chunk:
// it publishes the chunk's loads and the previous chunk's wave masks, whose
// union a lane of waves 0 and 4 then counts.
constexpr int kWorkStages = 3;
constexpr int kWorkStageBytes = kChunk * kHeadDim * 2;  // 8 KiB
constexpr int kWorkWaitOne = 0x0071;  // s_waitcnt vmcnt(1) lgkmcnt(0): also the wave-mask write

__global__ __launch_bounds__(512) void tile_work_kernel(TileOrderArgs a) {
  __shared__ __attribute__((aligned(16))) u16 stage[kWorkStages][kWorkStageBytes / 2];
  __shared__ uint32_t wmask[2][8];
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, r = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = blockIdx.y;
  const int qt = blockIdx.x * 2 + (wave >> 2);  // this wave's tile
  const int row = qt * kQTile + (wave & 3) * 32 + r;
  const bool valid = row < a.N;
  QFrag qf;
  load_qfrag(qf, a.q + (int64_t)h * a.N * kHeadDim, row, valid, g);
  float tau = __builtin_inff();
  if (valid) tau = make_tau(a.mu[(int64_t)h * a.N + row], a.sigma[(int64_t)h * a.N + row], a.beta);
  // the only loads the compiler tracks: drained here, so none of its waits
  // depends on the direct loads below
  __builtin_amdgcn_s_waitcnt(0);

  // direct loads: wave w fills 16-byte slots 64 w .. 64 w + 63 of a stage,
  // slot P holding chunk (P % 16) ^ (row % 16) of block row P / 16
  const int P = wave * 64 + lane, srow = P >> 4, sc = (P & 15) ^ (srow & 15);
  const u16* src = a.khi + ((int64_t)h * a.nb_pad + srow) * kHeadDim + sc * 8;
  const int n_chunks = a.nb_pad / kChunk;
  auto dma_chunk = [&](int c, int st) __attribute__((always_inline)) {
    c = c < n_chunks ? c : n_chunks - 1;  // past the end: a stage never read again
    dma_to_lds16(src + (int64_t)c * kChunk * kHeadDim, lds_addr(&stage[st][wave * 64 * 8]));
  };
  dma_chunk(0, 0);
  dma_chunk(1, 1);
  int work = 0;
  const bool counter = lane == 0 && (wave & 3) == 0;  // lane 0 of waves 0 and 4
  const int tbase = wave & 4;
  for (int c = 0; c < n_chunks; ++c) {
    __builtin_amdgcn_s_waitcnt(kWorkWaitOne);  // this wave's load of chunk c and its mask write landed
    __builtin_amdgcn_s_barrier();              // every wave's; stage of c - 1 read
    asm volatile("" ::: "memory");
    dma_chunk(c + 2, (c + 2) % kWorkStages);
    if (counter && c > 0) {
      const uint32_t* m = wmask[(c - 1) & 1] + tbase;
      work += __popc(m[0] | m[1] | m[2] | m[3]);
    }
    const u16* st = stage[c % kWorkStages];
    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8 hi = *reinterpret_cast<const bf16x8*>(st + (r * 16 + ((2 * ks + g) ^ (r & 15))) * 8);
      acc = mfma32(hi, qf.k[ks], acc);
    }
    const float scale = 0.08838834764831845f;  // 1/sqrt(128)
    const int b0 = c * kChunk;
    // the wave's union per block: each lane's selections as a bit mask (element
    // i is block acc_row(i, 0) + 4g; invalid rows have tau = +inf and select
    // nothing), OR-ed over the wave
    uint32_t bits = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      bits |= is_selected(acc[i] * scale, tau) ? 1u << acc_row(i, 0) : 0u;
    uint32_t mine = wave_or(bits << (4 * g));
    const int left = a.nb - b0;  // blocks of this chunk that exist
    if (left < 32) mine &= (1u << left) - 1u;
    if (lane == 0) wmask[c & 1][wave] = mine;
  }
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  if (counter && qt < a.n_qt) {
    const uint32_t* m = wmask[(n_chunks - 1) & 1] + tbase;
    work += __popc(m[0] | m[1] | m[2] | m[3]);
    a.work[(int64_t)h * a.n_qt + qt] = work;
  }
}

// tile_order_kernel: one workgroup per head.  Tile i's rank is the number of
// tiles with more work, or as much work and a smaller index; the tile of rank
// r runs as the head's r-th workgroup.
__global__ __launch_bounds__(1024) void tile_order_kernel(TileOrderArgs a) {
  __shared__ int work[kOrderMaxTiles];
  const int h = blockIdx.x, n = a.n_qt;
  for (int i = threadIdx.x; i < n; i += 1024) work[i] = a.work[(int64_t)h * n + i];
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += 1024) {
    const int w = work[i];
    int rank = 0;
    for (int j = 0; j < n; ++j) {
      const int wj = work[j];
      rank += (wj > w) | ((wj == w) & (j < i));
    }
    a.order[(int64_t)h * n + rank] = h * n + i;
  }
}

hipError_t launch_tile_order(const TileOrderArgs& a, hipStream_t s) {
  if (a.n_qt > kOrderMaxTiles) return hipErrorInvalidValue;
  const hipError_t e = launch_kernel(tile_work_kernel, dim3((a.n_qt + 1) / 2, a.H), dim3(512), s, a);
  if (e != hipSuccess) return e;
  return launch_kernel(tile_order_kernel, dim3(a.H), dim3(1024), s, a);
}

// ---------------------------------------------------------------------------
// Inspection: proxy scores of a row range.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void proxy_kernel(ProxyArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 5;
  const int h = blockIdx.y;
  const int rl = blockIdx.x * kQTile + wave * 32 + (lane & 31);  // local row
  const int row = a.row0 + rl;
  const bool valid = rl < a.nrows && row < a.N;
  QFrag qf;
  load_qfrag(qf, a.q + (int64_t)h * a.N * kHeadDim, row, valid, g);
  const float* kb = a.kbar + (int64_t)h * a.nb * kHeadDim;
  for (int b0 = 0; b0 < a.nb; b0 += kChunk) {
    f32x16 p = proxy_chunk(qf, kb, b0, a.nb, lane);
    if (!valid) continue;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      int blk = b0 + acc_row(i, g);
      if (blk < a.nb) a.p[((int64_t)h * a.nrows + rl) * a.nb + blk] = p[i];
    }
  }
}

hipError_t launch_proxy(const ProxyArgs& a, hipStream_t s) {
  dim3 grid((a.nrows + kQTile - 1) / kQTile, a.H);
  return launch_kernel(proxy_kernel, grid, dim3(256), s, a);
}

// ---------------------------------------------------------------------------
// Inspection: selection mask and density counts, with the forward kernel's
// predicate (same proxy_chunk, make_tau and is_selected).
// ---------------------------------------------------------------------------
__global__ void zero_counts_kernel(unsigned long long* c) {
  if (threadIdx.x < 4) c[threadIdx.x] = 0ull;
}

__global__ __launch_bounds__(256) void mask_kernel(MaskArgs a) {
  __shared__ uint32_t wmask[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 5;
  const int h = blockIdx.y;
  const int rl = blockIdx.x * kQTile + wave * 32 + (lane & 31);
  const int row = a.row0 + rl;
  const bool valid = rl < a.nrows && row < a.N;
  QFrag qf;
  load_qfrag(qf, a.q + (int64_t)h * a.N * kHeadDim, row, valid, g);
  const float* kb = a.kbar + (int64_t)h * a.nb * kHeadDim;
  float tau = __builtin_inff();
  if (valid) tau = make_tau(a.mu[(int64_t)h * a.N + row], a.sigma[(int64_t)h * a.N + row], a.beta);
  unsigned long long n_sel = 0, n_t32 = 0, n_t128 = 0, n_pairs = 0;
  for (int b0 = 0; b0 < a.nb; b0 += kChunk) {
    f32x16 p = proxy_chunk(qf, kb, b0, a.nb, lane);
    uint32_t mine = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      int off = acc_row(i, g);
      int blk = b0 + off;
      bool sel = valid && blk < a.nb && is_selected(p[i], tau);
      mine |= (uint32_t)sel << off;
      if (valid && blk < a.nb && a.mask)
        a.mask[((int64_t)h * a.nrows + rl) * a.nb + blk] = sel ? 1 : 0;
    }
    n_sel += __popc(mine);
    uint32_t wu = mine;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) wu |= __shfl_xor(wu, o);
    __syncthreads();
    if (lane == 0) wmask[wave] = wu;
    __syncthreads();
    if (lane == 0) {
      n_t32 += __popc(wu);
      if (wave == 0) {
        uint32_t u = wmask[0] | wmask[1] | wmask[2] | wmask[3];
        n_t128 += __popc(u);
        n_pairs += min(kChunk, a.nb - b0);
      }
    }
  }
  // per-lane selected counts -> wave sum
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) n_sel += __shfl_xor(n_sel, o);
  if (lane == 0) {
    atomicAdd(&a.counts[0], n_sel);
    atomicAdd(&a.counts[1], n_t32);
    if (wave == 0) {
      atomicAdd(&a.counts[2], n_t128);
      atomicAdd(&a.counts[3], n_pairs);
    }
  }
}

hipError_t launch_mask(const MaskArgs& a, hipStream_t s) {
  const hipError_t e = launch_kernel(zero_counts_kernel, dim3(1), dim3(64), s, a.counts);
  if (e != hipSuccess) return e;
  dim3 grid((a.nrows + kQTile - 1) / kQTile, a.H);
  return launch_kernel(mask_kernel, grid, dim3(256), s, a);
}

}  // namespace solattn

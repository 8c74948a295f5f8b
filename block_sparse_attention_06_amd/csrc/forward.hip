// Fused attention forward for gfx950: dense softmax attention, and
// query-thresholded block-sparse attention with a first-order Taylor term for
// the rejected blocks, in one online-softmax pass.
//
// Sol-Engine LTX25 page, "Stage 2 Optimization -- Core Technology: Sol-Attn":
//  - routing is folded into the softmax pass: pooled keys are taken 32 blocks
//    at a time ("chunk-wise"), their proxy scores are compared with each row's
//    threshold, and only then are the chunk's key/value tiles fetched -- the
//    proxy scores of a chunk live in registers and are never stored;
//  - rejected blocks contribute n_j e^{mu_i} (1 + p_ij - mu_i) on the pooled
//    value (numerator) and the same weight (denominator).
// doubleAI page, "Attention across two GPUs": with few query tiles the key
// range is split over workgroups and the partial answers, each carrying its
// running maximum and denominator, are merged exactly (combine_kernel).
//
// Workgroup: 4 waves x 32 query rows = 128 rows of one head.  Per key tile the
// workgroup stages K (row-major) and V^T (transposed, keys permuted so an MFMA
// operand is one 16-byte LDS read) in LDS; each wave then computes
// S^T = K Q^T and O^T += V^T P^T on bf16 MFMA with fp32 accumulation.  A tile
// is fetched when any wave of the workgroup selected the block, and a wave
// issues its MFMAs only when one of its own 32 rows selected it; rows that did
// not select it are masked to -inf inside the tile.
#include "device.hpp"
#include "launch.hpp"

namespace solattn {

template <bool SPARSE, int KB>
__global__ __launch_bounds__(256, 2) void fwd_kernel(FwdArgs a) {
  constexpr int KS = kHeadDim + 8;  // K tile row stride (bf16 elements)
  constexpr int VS = KB + 8;        // V^T tile row stride
  constexpr int NT = KB / 32;       // 32-key sub-tiles
  __shared__ __attribute__((aligned(16))) u16 Ks[KB * KS];
  __shared__ __attribute__((aligned(16))) u16 Vt[kHeadDim * VS];
  __shared__ uint32_t wmask[2][4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5, r32 = lane & 31;

  // Workgroups are dealt to the 8 XCDs round-robin; give each XCD a contiguous
  // run of (head, query tile, split) so the workgroups sharing an L2 read the
  // same head's keys and values.
  const int per_xcd = gridDim.x >> 3;
  const int logical = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (logical >= a.total) return;
  const int split = logical % a.splits;
  const int tq = logical / a.splits;
  const int qt = tq % a.n_qt, h = tq / a.n_qt;
  const int row = qt * kQTile + wave * 32 + r32;
  const bool qvalid = row < a.N;

  QFrag qf;
  load_qfrag(qf, a.q + (int64_t)h * a.N * kHeadDim, row, qvalid, g);
  const u16* kh = a.k + (int64_t)h * a.Nk * kHeadDim;
  const u16* vh = a.v + (int64_t)h * a.Nk * kHeadDim;

  const int t_begin = split * a.tiles_per_split;
  const int t_end = min(a.nb, t_begin + a.tiles_per_split);
  const float sl2 = 0.08838834764831845f * kLog2e;  // softmax scale in log2 units

  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
  float l = 0.f;   // this lane's share of the denominator, relative to 2^m
  float m;         // running maximum (log2 units)
  float mu = 0.f, tau = __builtin_inff();
  if constexpr (SPARSE) {
    if (qvalid) {
      mu = a.mu[(int64_t)h * a.N + row];
      tau = make_tau(mu, a.sigma[(int64_t)h * a.N + row], a.beta);
    }
    m = mu * kLog2e;  // the Taylor terms are relative to e^mu: start the reference there
  } else {
    m = -__builtin_inff();
  }

  // ---- stage one key tile (K row-major, V transposed) in LDS ----
  auto load_tile = [&](int tile) {
    const int key0 = tile * KB;
#pragma unroll
    for (int rep = 0; rep < KB / 16; ++rep) {
      const int u = tid + 256 * rep, r = u >> 4, c = u & 15;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (key0 + r < a.Nk)
        x = *reinterpret_cast<const u32x4*>(kh + (int64_t)(key0 + r) * kHeadDim + c * 8);
      *reinterpret_cast<u32x4*>(&Ks[r * KS + c * 8]) = x;
    }
#pragma unroll
    for (int rep = 0; rep < KB / 64; ++rep) {
      const int u = tid + 256 * rep, c = u & 15, quad = u >> 4;
      u32x4 x[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = key0 + quad * 4 + r;
        x[r] = u32x4{0u, 0u, 0u, 0u};
        if (key < a.Nk) x[r] = *reinterpret_cast<const u32x4*>(vh + (int64_t)key * kHeadDim + c * 8);
      }
      const int qq = quad & 3;
      const int col = (quad >> 2) * 16 + (qq & 1) * 8 + (qq >> 1) * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        u32x2 lo, hi;
        lo[0] = (x[0][e] & 0xffffu) | (x[1][e] << 16);
        lo[1] = (x[2][e] & 0xffffu) | (x[3][e] << 16);
        hi[0] = (x[0][e] >> 16) | (x[1][e] & 0xffff0000u);
        hi[1] = (x[2][e] >> 16) | (x[3][e] & 0xffff0000u);
        *reinterpret_cast<u32x2*>(&Vt[(c * 8 + 2 * e) * VS + col]) = lo;
        *reinterpret_cast<u32x2*>(&Vt[(c * 8 + 2 * e + 1) * VS + col]) = hi;
      }
    }
  };

  // ---- exact online-softmax update with one staged tile ----
  auto compute_tile = [&](int tile, bool mine) {
    f32x16 s[NT];
#pragma unroll
    for (int kt = 0; kt < NT; ++kt) {
      s[kt] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        u32x4 ka = *reinterpret_cast<const u32x4*>(&Ks[(kt * 32 + r32) * KS + ks * 16 + g * 8]);
        s[kt] = mfma32(as_bf16x8(ka), qf.k[ks], s[kt]);
      }
    }
    const int key0 = tile * KB;
    float mx = -__builtin_inff();
#pragma unroll
    for (int kt = 0; kt < NT; ++kt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = key0 + kt * 32 + acc_row(i, g);
        const float x = (mine && key < a.Nk) ? s[kt][i] * sl2 : -__builtin_inff();
        s[kt][i] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mn = fmaxf(m, mx);
    const float mref = mn == -__builtin_inff() ? 0.f : mn;
    const float alpha = fast_exp2(m - mref);
    m = mn;
    l *= alpha;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
    bf16x8 pb[NT * 2];
    float rs = 0.f;
#pragma unroll
    for (int kt = 0; kt < NT; ++kt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pe = fast_exp2(s[kt][i] - mref);
        rs += pe;
        pb[kt * 2 + (i >> 3)][i & 7] = (__bf16)pe;
      }
    }
    l += rs;
#pragma unroll
    for (int kt = 0; kt < NT; ++kt) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          u32x4 va = *reinterpret_cast<const u32x4*>(
              &Vt[(dt * 32 + r32) * VS + kt * 32 + h2 * 16 + g * 8]);
          o[dt] = mfma32(as_bf16x8(va), pb[kt * 2 + h2], o[dt]);
        }
      }
    }
  };

  if constexpr (SPARSE) {
    const float* kb = a.kbar + (int64_t)h * a.nb * kHeadDim;
    const u16* vsum = a.vsumT + (int64_t)h * kHeadDim * a.nb_pad;
    int parity = 0;
    for (int c0 = t_begin; c0 < t_end; c0 += kChunk, parity ^= 1) {
      // routing: proxy scores of this chunk, selection, Taylor weights
      const f32x16 p = proxy_chunk(qf, kb, c0, a.nb, lane);
      const float f = fast_exp2(mu * kLog2e - m);  // e^{mu - M}: Taylor terms at the current reference
      uint32_t mine = 0;
      // Weights of the rejected blocks enter the MFMA as bf16 hi + lo parts:
      // when many blocks share nearly the same weight, a single bf16 rounding
      // would bias the Taylor mass coherently instead of averaging out.
      bf16x8 whi[2], wlo[2];
      float wden = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int off = acc_row(i, g);
        const int blk = c0 + off;
        const bool inr = qvalid && blk < t_end;
        const bool sel = inr && is_selected(p[i], tau);
        mine |= (uint32_t)sel << off;
        const float wt = (inr && !sel) ? (1.f + p[i] - mu) * f : 0.f;
        const __bf16 wh = (__bf16)wt;
        whi[i >> 3][i & 7] = wh;
        wlo[i >> 3][i & 7] = (__bf16)(wt - (float)wh);
        const int nj = inr ? min(KB, a.Nk - blk * KB) : 0;
        wden = __builtin_fmaf((float)nj, wt, wden);
      }
      // Taylor part: O^T += (block sums of V)^T W^T over the chunk, on MFMA
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          u32x4 va = *reinterpret_cast<const u32x4*>(
              vsum + (int64_t)(dt * 32 + r32) * a.nb_pad + c0 + h2 * 16 + g * 8);
          o[dt] = mfma32(as_bf16x8(va), whi[h2], o[dt]);
          o[dt] = mfma32(as_bf16x8(va), wlo[h2], o[dt]);
        }
      }
      l += wden;
      // blocks wanted by this row, by this wave, by the workgroup
      const uint32_t full = mine | __shfl_xor(mine, 32);
      uint32_t wu = full;
#pragma unroll
      for (int sh = 1; sh < 32; sh <<= 1) wu |= __shfl_xor(wu, sh);
      if (lane == 0) wmask[parity][wave] = wu;
      __syncthreads();
      uint32_t todo = wmask[parity][0] | wmask[parity][1] | wmask[parity][2] | wmask[parity][3];
      while (todo) {
        const int bo = __builtin_ctz(todo);
        todo &= todo - 1;
        __syncthreads();
        load_tile(c0 + bo);
        __syncthreads();
        if ((wu >> bo) & 1u) compute_tile(c0 + bo, (full >> bo) & 1u);
      }
    }
  } else {
    for (int tile = t_begin; tile < t_end; ++tile) {
      __syncthreads();
      load_tile(tile);
      __syncthreads();
      compute_tile(tile, true);
    }
  }

  // ---- epilogue ----
  const float lt = l + __shfl_xor(l, 32);
  if (!qvalid) return;
  if (a.splits == 1) {
    const float inv = 1.f / lt;
    u16* orow = a.out + ((int64_t)h * a.N + row) * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        u32x2 pk;
        pk[0] = (uint32_t)f32_to_bf16_bits(o[dt][q4 * 4 + 0] * inv) |
                ((uint32_t)f32_to_bf16_bits(o[dt][q4 * 4 + 1] * inv) << 16);
        pk[1] = (uint32_t)f32_to_bf16_bits(o[dt][q4 * 4 + 2] * inv) |
                ((uint32_t)f32_to_bf16_bits(o[dt][q4 * 4 + 3] * inv) << 16);
        *reinterpret_cast<u32x2*>(orow + dt * 32 + q4 * 8 + g * 4) = pk;
      }
    }
    if (a.lse && g == 0) a.lse[(int64_t)h * a.N + row] = m * kLn2 + logf(lt);
  } else {
    const int64_t prow = ((int64_t)split * a.H + h) * a.N + row;
    float* po = a.part_o + prow * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        f32x4 v4 = {o[dt][q4 * 4], o[dt][q4 * 4 + 1], o[dt][q4 * 4 + 2], o[dt][q4 * 4 + 3]};
        *reinterpret_cast<f32x4*>(po + dt * 32 + q4 * 8 + g * 4) = v4;
      }
    }
    if (g == 0) {
      a.part_ml[prow * 2] = m;
      a.part_ml[prow * 2 + 1] = lt;
    }
  }
}

hipError_t launch_forward(const FwdArgs& a, bool sparse, int B, hipStream_t s) {
  const int grid = (a.total + 7) & ~7;
  if (!sparse)
    fwd_kernel<false, 128><<<grid, 256, 0, s>>>(a);
  else if (B == 64)
    fwd_kernel<true, 64><<<grid, 256, 0, s>>>(a);
  else
    fwd_kernel<true, 128><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Exact N-way merge of split partials (unnormalised numerator, max, denominator).
// One workgroup of 128 threads per (head, row); thread = dimension.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(128) void combine_kernel(CombineArgs a) {
  const int64_t rg = blockIdx.x;  // h * N + row
  const int64_t HN = (int64_t)a.H * a.N;
  const int d = threadIdx.x;
  float M = -__builtin_inff();
  for (int s = 0; s < a.splits; ++s) M = fmaxf(M, a.part_ml[(s * HN + rg) * 2]);
  const float mref = M == -__builtin_inff() ? 0.f : M;
  float num = 0.f, den = 0.f;
  for (int s = 0; s < a.splits; ++s) {
    const float w = exp2f(a.part_ml[(s * HN + rg) * 2] - mref);
    den += w * a.part_ml[(s * HN + rg) * 2 + 1];
    num += w * a.part_o[(s * HN + rg) * kHeadDim + d];
  }
  a.out[rg * kHeadDim + d] = f32_to_bf16_bits(num / den);
  if (d == 0 && a.lse) a.lse[rg] = mref * kLn2 + logf(den);
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  combine_kernel<<<(unsigned)((int64_t)a.H * a.N), 128, 0, s>>>(a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Two-way LSE merge (doubleAI page, "Attention across two GPUs").
// 16 threads per row, 8 dimensions (16 bytes) each; the 16 threads of a row
// sit in one wave, so a row is read before it is written when out aliases an
// input.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t rg = gid >> 4;
  const int c = (int)(gid & 15);
  if (rg >= (int64_t)a.H * a.N) return;
  const float la = a.lse_a[rg], lb = a.lse_b[rg];
  const float M = fmaxf(la, lb);
  float wa = 0.f, wb = 0.f, L = -__builtin_inff();
  if (M != -__builtin_inff()) {
    const float ea = expf(la - M), eb = expf(lb - M);
    const float z = ea + eb;
    L = M + logf(z);
    wa = ea / z;
    wb = eb / z;
  }
  const u32x4 xa = *reinterpret_cast<const u32x4*>(a.out_a + rg * kHeadDim + c * 8);
  const u32x4 xb = *reinterpret_cast<const u32x4*>(a.out_b + rg * kHeadDim + c * 8);
  u32x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float lo = wa * __uint_as_float(xa[e] << 16) + wb * __uint_as_float(xb[e] << 16);
    const float hi = wa * __uint_as_float(xa[e] & 0xffff0000u) + wb * __uint_as_float(xb[e] & 0xffff0000u);
    r[e] = (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
  }
  *reinterpret_cast<u32x4*>(a.out + rg * kHeadDim + c * 8) = r;
  if (c == 0) a.lse[rg] = L;
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t s) {
  const int64_t threads = (int64_t)a.H * a.N * 16;
  merge_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace solattn

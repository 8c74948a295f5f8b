// Fused attention forward for gfx950: dense softmax attention, and
// query-thresholded block-sparse attention with a first-order Taylor term for
// the rejected blocks, in one online-softmax pass.
//
// Sol-Engine LTX25 page, "Stage 2 Optimization -- Core Technology: Sol-Attn":
//  - routing is folded into the softmax pass: pooled keys are taken 32 blocks
//    at a time ("chunk-wise"), their proxy scores are compared with each row's
//    threshold, and only the selected blocks' key/value tiles are fetched --
//    the proxy scores of a chunk live in registers and are never stored;
//  - rejected blocks contribute n_j e^{mu_i} (1 + p_ij - mu_i) on the pooled
//    value (numerator) and the same weight (denominator).
// doubleAI page, "Attention across two GPUs": with few query tiles the key
// range is split over workgroups and the partial answers, each carrying its
// running maximum and denominator, are merged exactly (combine_kernel).
//
// Workgroup: 4 waves x 32 query rows = 128 rows of one head; two workgroups
// per CU.  Keys are processed in units of 64.  Each unit's K and V rows are
// staged in LDS row-major (XOR-swizzled 16-byte chunks), double-buffered: the
// next unit's global loads are issued into registers before the current unit
// is computed and written to the other LDS buffer after it, with one barrier
// per unit.  Each wave computes S^T = K Q^T and O^T += V^T P^T on bf16 MFMA
// (fp32 accumulation); the V^T operand comes straight from the row-major tile
// through the transposing LDS read.  A unit is fetched when any wave of the
// workgroup selected its block; a wave issues MFMAs only when one of its own
// 32 rows did, and rows that did not select it get zero probability.
#include "device.hpp"
#include "launch.hpp"

namespace solattn {

namespace {

constexpr int kUnit = 64;             // keys per staged unit
constexpr float kRescaleSlack = 8.f;  // log2 units the running reference may lag the max

// LDS layouts of one 64-key unit ([64 rows][128 bf16], 16-byte chunks):
// K rows put chunk c at c ^ (row % 16): the S operand reads 16 consecutive rows
// at one chunk per LDS cycle.  V rows put chunk c at c ^ 4 (row % 4): the
// transposing read takes 4 consecutive rows x 4 chunks per 16 lanes.
__device__ __forceinline__ int k_off(int row, int c) { return row * kHeadDim + ((c ^ (row & 15)) << 3); }
__device__ __forceinline__ int v_off(int row, int c) { return row * kHeadDim + ((c ^ ((row & 3) << 2)) << 3); }

}  // namespace

template <bool SPARSE, int KB>
__global__ __launch_bounds__(256, 2) void fwd_kernel(FwdArgs a) {
  __shared__ __attribute__((aligned(16))) u16 lds_k[2][kUnit * kHeadDim];
  __shared__ __attribute__((aligned(16))) u16 lds_v[2][kUnit * kHeadDim];
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
  const int Nk = a.Nk;

  const int t_begin = split * a.tiles_per_split;
  const int t_end = min(a.nb, t_begin + a.tiles_per_split);
  const float sl2 = 0.08838834764831845f * kLog2e;  // softmax scale in log2 units

  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
  float l = 0.f;  // this lane's share of the denominator, relative to 2^m
  float m;        // reference of the running sums (log2 units), within kRescaleSlack of the max
  float mu = 0.f, tau = __builtin_inff();
  if constexpr (SPARSE) {
    if (qvalid) {
      mu = gload<float>(a.mu + (int64_t)h * a.N + row);
      tau = make_tau(mu, gload<float>(a.sigma + (int64_t)h * a.N + row), a.beta);
    }
    m = mu * kLog2e;  // Taylor terms are relative to e^mu: start the reference there
  } else {
    m = -__builtin_inff();
  }

  // ---- staging: 64 rows x 16 chunks of K and of V, 4 + 4 chunks per thread ----
  u32x4 stg[8];
  // Rows past the last key re-read the last key (finite data): their scores are
  // masked and their probabilities are zero, so no load needs a predicate.
  auto issue_loads = [&](int key0) __attribute__((always_inline)) {
#pragma unroll
    for (int rep = 0; rep < 4; ++rep) {
      const int idx = tid + 256 * rep, r = idx >> 4, c = idx & 15;
      const int64_t off = (int64_t)min(key0 + r, Nk - 1) * kHeadDim + c * 8;
      stg[rep] = gload<u32x4>(kh + off);
      stg[4 + rep] = gload<u32x4>(vh + off);
    }
  };
  auto write_lds = [&](int st) __attribute__((always_inline)) {
#pragma unroll
    for (int rep = 0; rep < 4; ++rep) {
      const int idx = tid + 256 * rep, r = idx >> 4, c = idx & 15;
      *reinterpret_cast<u32x4*>(&lds_k[st][k_off(r, c)]) = stg[rep];
      *reinterpret_cast<u32x4*>(&lds_v[st][v_off(r, c)]) = stg[4 + rep];
    }
  };

  // ---- exact online-softmax update with one staged unit ----
  auto compute = [&](int st, int key0, bool mine) __attribute__((always_inline)) {
    f32x16 s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      s[kt] = f32x16{};
      const int r = kt * 32 + r32;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const u32x4 ka = *reinterpret_cast<const u32x4*>(&lds_k[st][k_off(r, ks * 2 + g)]);
        s[kt] = mfma32(as_bf16x8(ka), qf.k[ks], s[kt]);
      }
    }
    if (key0 + kUnit > Nk) {  // ragged last unit: keys past the end do not exist
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (key0 + kt * 32 + acc_row(i, g) >= Nk) s[kt][i] = -__builtin_inff();
    }
    float mx = -__builtin_inff();
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kt][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mc = mx * sl2;
    // move the reference only when the max outruns it by more than the slack
    const bool up = mine && (mc > m + kRescaleSlack);
    if (__ballot(up)) {
      const float alpha = up ? fast_exp2(m - mc) : 1.f;
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
    }
    if (up) m = mc;
    const float neg_ref = mine ? -m : -__builtin_inff();  // rows that did not select: p = 0
    bf16x8 pb[4];
    float rs = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pe = fast_exp2(__builtin_fmaf(s[kt][i], sl2, neg_ref));
        rs += pe;
        pb[kt * 2 + (i >> 3)][i & 7] = (__bf16)pe;
      }
    }
    l += rs;
    // O^T += V^T P^T: the V^T operand of k-step (kt, h2) holds keys
    // kt*32 + h2*16 + {4g..4g+3, 8+4g..8+4g+3} -- the keys of P that this lane
    // half holds -- read as two transposed 4 x 16 blocks per 16-lane group.
    const int G = lane >> 4, j = lane & 15;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int r0 = kt * 32 + h2 * 16 + g * 4 + (j >> 2);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const int col = dt * 32 + (G & 1) * 16 + 4 * (j & 3);
          const u32x2 v0 = lds_read_tr16(&lds_v[st][v_off(r0, col >> 3) + (col & 7)]);
          const u32x2 v1 = lds_read_tr16(&lds_v[st][v_off(r0 + 8, col >> 3) + (col & 7)]);
          const u32x4 va = {v0[0], v0[1], v1[0], v1[1]};
          o[dt] = mfma32(as_bf16x8(va), pb[kt * 2 + h2], o[dt]);
        }
      }
    }
  };

  // ---- the stream of units: key offset, and whether this row / this wave take it ----
  struct Unit {
    int key0;
    bool mine, need;
  };

  if constexpr (SPARSE) {
    const u16* khi = a.khi + (int64_t)h * a.nb_pad * kHeadDim;
    const u16* klo = a.klo + (int64_t)h * a.nb_pad * kHeadDim;
    const u16* vsum = a.vsumT + (int64_t)h * kHeadDim * a.nb_pad;
    // Route one chunk of 32 blocks: proxy scores, selection, Taylor part of
    // the rejected blocks (at the current reference m).  Returns the blocks any
    // row of the workgroup selected; `full` = this row's, `wv` = this wave's.
    auto route = [&](int c0, int parity, uint32_t& full, uint32_t& wv)
        __attribute__((always_inline)) -> uint32_t {
      const f32x16 p = proxy_chunk_hl(qf, khi, klo, c0, lane);
      const float f = fast_exp2(mu * kLog2e - m);  // e^{mu} relative to the reference
      uint32_t mine = 0;
      // Weights enter the MFMA as bf16 hi + lo parts: when many blocks share
      // nearly the same weight, a single bf16 rounding would bias the Taylor
      // mass coherently instead of averaging out.
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
        __bf16 wh, wl;
        split_bf16(wt, wh, wl);
        whi[i >> 3][i & 7] = wh;
        wlo[i >> 3][i & 7] = wl;
        const int nj = inr ? min(KB, Nk - blk * KB) : 0;
        wden = __builtin_fmaf((float)nj, wt, wden);
      }
      // Taylor part: O^T += (block sums of V)^T W^T over the chunk, on MFMA
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const u32x4 va = gload<u32x4>(vsum + (int64_t)(dt * 32 + r32) * a.nb_pad + c0 + h2 * 16 + g * 8);
          o[dt] = mfma32(as_bf16x8(va), whi[h2], o[dt]);
          o[dt] = mfma32(as_bf16x8(va), wlo[h2], o[dt]);
        }
      }
      l += wden;
      full = mine | __shfl_xor(mine, 32);
      uint32_t w = full;
#pragma unroll
      for (int sh = 1; sh < 32; sh <<= 1) w |= __shfl_xor(w, sh);
      wv = w;
      if (lane == 0) wmask[parity][wave] = w;
      __syncthreads();
      return wmask[parity][0] | wmask[parity][1] | wmask[parity][2] | wmask[parity][3];
    };

    // chunk A is being consumed; chunk B (the next one) is already routed
    int cA = t_begin, cB = t_begin + kChunk;
    uint32_t fullA, wvA, fullB = 0, wvB = 0, UB = 0;
    uint32_t UA = route(cA, 0, fullA, wvA);
    if (cB < t_end) UB = route(cB, 1, fullB, wvB);
    int pend = -1;  // second half of a 128-key block still to come
    bool pend_mine = false, pend_need = false;
    auto next = [&](Unit& u) __attribute__((always_inline)) -> bool {
      if (KB == 128 && pend >= 0) {
        u = Unit{pend, pend_mine, pend_need};
        pend = -1;
        return true;
      }
      while (true) {
        if (UA) {
          const int b = __builtin_ctz(UA);
          UA &= UA - 1;
          u = Unit{(cA + b) * KB, ((fullA >> b) & 1u) != 0, ((wvA >> b) & 1u) != 0};
          if (KB == 128) {
            pend = u.key0 + kUnit;
            pend_mine = u.mine;
            pend_need = u.need;
          }
          return true;
        }
        if (cB >= t_end) return false;
        cA = cB;
        UA = UB;
        fullA = fullB;
        wvA = wvB;
        cB += kChunk;
        UB = 0;
        if (cB < t_end) UB = route(cB, ((cB - t_begin) / kChunk) & 1, fullB, wvB);
      }
    };

    Unit cur, nxt;
    bool have = next(cur);
    int st = 0;
    if (have) {
      issue_loads(cur.key0);
      write_lds(0);
    }
    __builtin_amdgcn_s_waitcnt(0);  // as in the dense loop: nothing outstanding at loop entry
    __syncthreads();
    while (have) {
      const bool hn = next(nxt);
      if (hn) issue_loads(nxt.key0);
      if (cur.need) compute(st, cur.key0, cur.mine);
      if (hn) write_lds(st ^ 1);
      __syncthreads();
      st ^= 1;
      cur = nxt;
      have = hn;
    }
  } else {
    const int u_begin = t_begin * (KB / kUnit);
    const int u_end = min(t_end * (KB / kUnit), (Nk + kUnit - 1) / kUnit);
    int st = 0;
    if (u_begin < u_end) {
      issue_loads(u_begin * kUnit);
      write_lds(0);
    }
    // Drain every load issued so far (query fragment included) on all paths, so
    // the loop's only outstanding loads are the prefetches its LDS writes wait for.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int u = u_begin; u < u_end; ++u) {
      const bool hn = u + 1 < u_end;
      if (hn) issue_loads((u + 1) * kUnit);
      compute(st, u * kUnit, true);
      if (hn) write_lds(st ^ 1);
      __syncthreads();
      st ^= 1;
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

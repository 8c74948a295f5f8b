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
// per CU.  Keys stream through LDS in units of 32 rows of K and V, in a ring of
// five stages filled by direct global->LDS loads four units ahead of the unit
// being computed (no registers hold data in flight; each wave waits only for
// its own loads of the next unit, then one barrier per unit publishes it).
// Rows sit row-major with XOR-swizzled 16-byte chunks.  Each wave computes
// S^T = K Q^T and O^T += V^T P^T on bf16 MFMA (fp32 accumulation); the V^T
// operand comes straight from the row-major tile through the transposing LDS
// read.  A unit is fetched when any wave of the workgroup selected its block;
// a wave issues MFMAs only when one of its own 32 rows did, and rows that did
// not select it get zero probability.
#include "device.hpp"
#include "launch.hpp"

namespace solattn {

namespace {

constexpr int kUnit = 32;                        // keys per staged unit
constexpr int kStageElems = kUnit * kHeadDim;    // bf16 per tensor per stage
constexpr float kRescaleSlack = 8.f;             // log2 units the reference may lag the max

// LDS layouts of a unit ([32 rows][128 bf16], 16-byte chunks): K rows put
// chunk c at c ^ (row % 16), so the S operand reads 16 consecutive rows at one
// chunk without bank conflicts; V rows put chunk c at c ^ 4 (row % 4), so the
// transposing read of 4 consecutive rows x 4 chunks per 16 lanes is
// conflict-free.
__device__ __forceinline__ int k_slot(int row, int c) { return c ^ (row & 15); }
__device__ __forceinline__ int v_slot(int row, int c) { return c ^ ((row & 3) << 2); }

// LDS ring depth.  Four-wave workgroups run two per CU and share 160 KiB:
// five 16 KiB stages each (loads four units ahead).  Eight-wave workgroups run
// one per CU and use eight stages (seven units ahead).
template <bool SPARSE, int WAVES>
constexpr int stages() { return WAVES == 8 ? 8 : 5; }

// s_waitcnt immediate (gfx9 encoding) for vmcnt(n) alone.
constexpr int vm_wait(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

// Each wave issues 16 / WAVES loads per unit; waiting until only the loads of
// the stages - 2 later units are in flight means this wave's loads of the next
// unit have landed.
template <bool SPARSE, int WAVES>
constexpr int wait_next_unit() { return vm_wait((16 / WAVES) * (stages<SPARSE, WAVES>() - 2)); }
constexpr int kWaitLgkm0 = 0xC07F;

__device__ __forceinline__ float partner(float x, int g) {
  // value of lane l ^ 32
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(g ? r[0] : r[1]);
}

__device__ __forceinline__ uint32_t partner_u(uint32_t x, int g) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return g ? r[0] : r[1];
}

}  // namespace

template <bool SPARSE, int KB, int WAVES>
__global__ __launch_bounds__(64 * WAVES, 2) void fwd_kernel(FwdArgs a) {
  constexpr int kStages = stages<SPARSE, WAVES>();
  constexpr int kWaitNext = wait_next_unit<SPARSE, WAVES>();
  constexpr int kRowsPerWave = kUnit / WAVES;  // unit rows each wave loads
  __shared__ __attribute__((aligned(16))) u16 lds_k[kStages][kStageElems];
  __shared__ __attribute__((aligned(16))) u16 lds_v[kStages][kStageElems];

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, r32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // Natural order: consecutive workgroups take consecutive query tiles of one
  // head and are dealt to the 8 XCDs round-robin, so all XCDs work on the same
  // one or two heads at a time and those heads' keys and values stay in the
  // memory-side cache.
  const int logical = blockIdx.x;
  if (logical >= a.total) return;
  const int split = logical % a.splits;
  const int tq = logical / a.splits;
  const int qt = tq % a.n_qt, h = tq / a.n_qt;
  const int row = qt * (32 * WAVES) + wave * 32 + r32;
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

  // The query fragment and row statistics are the only loads the compiler
  // tracks; drain them here so that no wait it places later also waits for
  // the key/value prefetches below (which it does not track).
  __builtin_amdgcn_s_waitcnt(0);

  // ---- direct global -> LDS loads of one unit: wave w fills K and V rows
  // w*32/WAVES onwards, four rows (1 KiB) per instruction; lane l lands in chunk slot
  // l % 16 of row l / 16 and fetches the global chunk that slot holds.
  // Rows past the last key re-read the last key (finite data): their scores
  // are masked and their probabilities are zero.
  auto dma_unit = [&](int key0, int st) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kRowsPerWave / 4; ++i) {
      const int r0 = wave * kRowsPerWave + i * 4;
      const int r = r0 + (lane >> 4), slot = lane & 15;
      const int64_t key = min(key0 + r, Nk - 1);
      dma_to_lds16(kh + key * kHeadDim + (k_slot(r, slot) << 3), lds_addr(&lds_k[st][r0 * kHeadDim]));
      dma_to_lds16(vh + key * kHeadDim + (v_slot(r, slot) << 3), lds_addr(&lds_v[st][r0 * kHeadDim]));
    }
  };

  // ---- exact online-softmax update with one staged unit ----
  auto compute = [&](int st, int key0, bool mine) __attribute__((always_inline)) {
    f32x16 s = {};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const u32x4 ka = *reinterpret_cast<const u32x4*>(
          &lds_k[st][r32 * kHeadDim + (k_slot(r32, ks * 2 + g) << 3)]);
      s = mfma32(as_bf16x8(ka), qf.k[ks], s);
    }
    if (key0 + kUnit > Nk) {  // ragged last unit: keys past the end do not exist
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (key0 + acc_row(i, g) >= Nk) s[i] = -__builtin_inff();
    }
    float mx = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
    mx = fmaxf(mx, partner(mx, g));
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
    bf16x8 pb[2];
#pragma unroll
    for (int i = 0; i < 16; ++i)
      pb[i >> 3][i & 7] = (__bf16)fast_exp2(__builtin_fmaf(s[i], sl2, neg_ref));
    // Row sum of the bf16 probabilities (the values the PV product uses), two
    // per instruction: dot(p_pair, (1, 1)) accumulated in fp32.
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 one2 = {(__bf16)1.f, (__bf16)1.f};
    float rsum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bf16x2 pr = {pb[t][2 * e], pb[t][2 * e + 1]};
        rsum[e] = __builtin_amdgcn_fdot2_f32_bf16(pr, one2, rsum[e], false);
      }
    l += (rsum[0] + rsum[1]) + (rsum[2] + rsum[3]);
    // O^T += V^T P^T: the V^T operand of k-step h2 holds keys
    // h2*16 + {4g..4g+3, 8+4g..8+4g+3} -- the keys of P this lane half holds --
    // read as two transposed 4 x 16 blocks per 16-lane group.
    const int G = lane >> 4, j = lane & 15;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int r0 = h2 * 16 + g * 4 + (j >> 2);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const int col = dt * 32 + (G & 1) * 16 + 4 * (j & 3);
        const u32x2 v0 = lds_read_tr16(&lds_v[st][r0 * kHeadDim + (v_slot(r0, col >> 3) << 3) + (col & 7)]);
        const u32x2 v1 = lds_read_tr16(&lds_v[st][(r0 + 8) * kHeadDim + (v_slot(r0 + 8, col >> 3) << 3) + (col & 7)]);
        const u32x4 va = {v0[0], v0[1], v1[0], v1[1]};
        o[dt] = mfma32(as_bf16x8(va), pb[h2], o[dt]);
      }
    }
  };

  // ---- one loop: iteration t issues the loads of unit t into stage t % S and
  // computes unit t - A (A = S - 1), issued A iterations earlier.  Unit slots
  // shift by one per iteration, so every index is static.  Once the stream is
  // exhausted, iterations load key 0 into a stage nobody reads (keeping the
  // count of loads in flight exact) until the last unit is computed.
  constexpr int A = kStages - 1;
  int qkey[A + 1];
  bool qmine[A + 1], qneed[A + 1], qval[A + 1];
#pragma unroll
  for (int i = 0; i <= A; ++i) {
    qkey[i] = 0;
    qmine[i] = qneed[i] = qval[i] = false;
  }
  int st_issue = 0;
  bool stream_done = false;

  // unit sources
  int u_next = t_begin * (KB / kUnit);                                 // dense
  const int u_end = min(t_end * (KB / kUnit), (Nk + kUnit - 1) / kUnit);
  int c_next = t_begin, cA = 0;                                        // sparse
  uint32_t UA = 0, fullA = 0, wvA = 0;
  int pend_left = 0, pend_key = 0;
  bool pend_mine = false, pend_need = false;
  const u16* khi = SPARSE ? a.khi + (int64_t)h * a.nb_pad * kHeadDim : nullptr;
  const u16* klo = SPARSE ? a.klo + (int64_t)h * a.nb_pad * kHeadDim : nullptr;
  const u16* vsum = SPARSE ? a.vsumT + (int64_t)h * kHeadDim * a.nb_pad : nullptr;

  while (true) {
    // -- next unit of the stream --
    bool have = false;
    int key0 = 0;
    bool mi = false, ne = false;
    if (!stream_done) {
      if constexpr (SPARSE) {
        if (pend_left == 0) {
          // Route chunks of 32 blocks until one has a selected block: proxy
          // scores, selection, and the Taylor part of the rejected blocks (at
          // the current reference m).  Any row of the workgroup selecting a
          // block makes the block a unit source; `fullA` = this row's
          // selections, `wvA` = this wave's.
          while (UA == 0 && c_next < t_end) {
            const int c0 = c_next;
            const f32x16 p = proxy_chunk_hl(qf, khi, klo, c0, lane);
            const float f = fast_exp2(mu * kLog2e - m);  // e^{mu} relative to the reference
            uint32_t sel_bits = 0;
            // Weights enter the MFMA as bf16 hi + lo parts: when many blocks
            // share nearly the same weight, a single bf16 rounding would bias
            // the Taylor mass coherently instead of averaging out.
            bf16x8 whi[2], wlo[2];
            float wden = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int off = acc_row(i, g);
              const int blk = c0 + off;
              const bool inr = qvalid && blk < t_end;
              const bool sel = inr && is_selected(p[i], tau);
              sel_bits |= (uint32_t)sel << off;
              const float wt = (inr && !sel) ? (1.f + p[i] - mu) * f : 0.f;
              __bf16 wh, wl;
              split_bf16(wt, wh, wl);
              whi[i >> 3][i & 7] = wh;
              wlo[i >> 3][i & 7] = wl;
              const int nj = inr ? min(KB, Nk - blk * KB) : 0;
              wden = __builtin_fmaf((float)nj, wt, wden);
            }
            // Taylor part: O^T += (block sums of V)^T W^T over the chunk, on MFMA
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
              for (int dt = 0; dt < 4; ++dt) {
                const u32x4 va =
                    gload<u32x4>(vsum + (int64_t)(dt * 32 + r32) * a.nb_pad + c0 + h2 * 16 + g * 8);
                o[dt] = mfma32(as_bf16x8(va), whi[h2], o[dt]);
                o[dt] = mfma32(as_bf16x8(va), wlo[h2], o[dt]);
              }
            }
            l += wden;
            fullA = sel_bits | partner_u(sel_bits, g);
            uint32_t w = fullA;
#pragma unroll
            for (int sh = 1; sh < 32; sh <<= 1) w |= __shfl_xor(w, sh);
            wvA = w;
            // Exchange the wave masks through the last bytes of the K tile of
            // the stage about to be refilled: nothing reads it until the unit
            // issued next lands, and the second barrier keeps every read of the
            // masks ahead of that refill.
            uint32_t* wmask = reinterpret_cast<uint32_t*>(&lds_k[st_issue][kStageElems - 2 * WAVES]);
            if (lane == 0) wmask[wave] = w;
            __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
            __builtin_amdgcn_s_barrier();
            uint32_t un = 0;
#pragma unroll
            for (int i = 0; i < WAVES; ++i) un |= wmask[i];
            UA = un;
            __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
            __builtin_amdgcn_s_barrier();
            cA = c0;
            c_next += kChunk;
          }
          if (UA) {
            const int b = __builtin_ctz(UA);
            UA &= UA - 1;
            pend_key = (cA + b) * KB;
            pend_left = KB / kUnit;
            pend_mine = ((fullA >> b) & 1u) != 0;
            pend_need = ((wvA >> b) & 1u) != 0;
          }
        }
        if (pend_left > 0) {
          have = true;
          key0 = pend_key;
          mi = pend_mine;
          ne = pend_need;
          pend_key += kUnit;
          --pend_left;
        }
      } else {
        if (u_next < u_end) {
          have = true;
          key0 = u_next * kUnit;
          mi = ne = true;
          ++u_next;
        }
      }
      stream_done = !have;
    }
    bool pending = false;  // units issued but not yet computed
#pragma unroll
    for (int i = 1; i <= A; ++i) pending |= qval[i];
    if (stream_done && !pending) break;

    // -- issue unit t, shift the slots, compute unit t - A --
    dma_unit(key0, st_issue);
#pragma unroll
    for (int i = 0; i < A; ++i) {
      qkey[i] = qkey[i + 1];
      qmine[i] = qmine[i + 1];
      qneed[i] = qneed[i + 1];
      qval[i] = qval[i + 1];
    }
    qkey[A] = key0;
    qmine[A] = mi;
    qneed[A] = ne;
    qval[A] = have;
    const int st_comp = st_issue == kStages - 1 ? 0 : st_issue + 1;
    st_issue = st_comp;
    if (qval[0] && qneed[0]) compute(st_comp, qkey[0], qmine[0]);
    __builtin_amdgcn_s_waitcnt(kWaitNext);  // this wave's loads of the next unit landed
    __builtin_amdgcn_s_barrier();           // ... and every wave's; its stage is free to refill
  }
  __builtin_amdgcn_s_waitcnt(0);  // no load may land after the workgroup ends

  // ---- epilogue ----
  const float lt = l + partner(l, g);
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

// Dense attention only: the sparse path runs fwd4_kernel.
hipError_t launch_forward(const FwdArgs& a, bool sparse, int B, hipStream_t s) {
  (void)B;
  if (sparse) return hipErrorInvalidValue;
  const int grid = (a.total + 7) & ~7;
  fwd_kernel<false, 128, 4><<<grid, 256, 0, s>>>(a);
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

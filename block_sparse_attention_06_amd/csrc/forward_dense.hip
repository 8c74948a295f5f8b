// Dense attention forward for gfx950: plain softmax attention in one online
// pass -- the dense mode of the forward entry point (and its sparse mode at
// beta = -inf), the split-key partials of short query sets, and dense key
// shares.  The query-thresholded sparse method runs in fwd_kernel.
//
// doubleAI page, "Attention across two GPUs": with few query tiles the key
// range is split over workgroups and the partial answers, each carrying its
// running maximum and denominator, are merged exactly (combine_kernel).
//
// Each wave owns 32 query rows, and every SIMD holds three waves: while one
// runs its softmax on the vector unit, another issues matrix products (at most
// 168 registers per lane).  Keys stream through LDS in units of 32 rows of K
// and V, each unit filled by direct global->LDS loads from four waves.  Two forms:
//
//  - W = 4: 128 query rows per workgroup, three workgroups per CU (48 KiB of
//    LDS each), a ring of three stages, one unit per iteration: iteration i
//    issues the loads of unit i + 2 into the stage unit i - 1 left (free since
//    the barrier that ended iteration i - 1), then computes S^T = K Q^T of
//    unit i, its online softmax and O^T += V^T P^T, and waits for its own
//    loads of unit i + 1; one barrier per unit publishes them.  Short query
//    sets (key splits) and small calls use it.
//  - W = 12: 384 query rows per workgroup, one workgroup per CU (96 KiB), a
//    ring of six stages, two units per iteration and barrier, loads four units
//    ahead, the two units of a pair loaded by waves 0-3 and 4-7.  Each staged unit feeds twelve waves instead of four, so a third
//    of the L2->LDS traffic of the W = 4 form crosses the chip for the same
//    products; on this power-limited part that buys clock (4K dense 0.7-2 %
//    faster on two boxes).  Long sequences use it.
//
// Against a pipelined loop at two workgroups per CU (each wave overlapping the
// softmax of one unit with the products of the next) and an 8-wave ping-pong
// schedule, the third wave per SIMD does the overlapping instead: 4K dense
// 234.8 vs 248.2 ms on one box, stage-2 8.97 vs 9.77 ms (W = 4 form).
#include "device.hpp"
#include "launch.hpp"

namespace solattn {

namespace {

constexpr int kDU = 32;                  // keys per staged unit
constexpr int kDUE = kDU * kHeadDim;     // bf16 per tensor per stage
constexpr int kDTile = 128;              // keys per split tile
// The running sums' reference may lag a row's maximum by up to 8 (log2
// units): a lane's row sum of one unit's probabilities stays within 2^8.
constexpr float kDSlackSum = 256.f;
// Workgroups of the W = 12 form that fill the chip once (one per CU).
constexpr int kDWideMinWGs = 256;

// Per form: units per iteration P and ring stages 3P.  A loading wave issues
// the 4 loads of one unit per iteration (W = 4: every wave, its quarter of the
// unit; W = 12: waves 0-3 the first unit of the pair, waves 4-7 the second),
// so vmcnt(4) at the end of an iteration leaves this iteration's unit in
// flight and has the one issued an iteration earlier landed.
template <int W> struct DenseForm {
  static constexpr int P = W == 4 ? 1 : 2;
  static constexpr int kRing = 3 * P;
  static constexpr int kWait = 0x0F74;  // s_waitcnt vmcnt(4)
  static constexpr int kRows = 32 * W;
};

}  // namespace

template <int W>
__global__ __launch_bounds__(64 * W, W == 4 ? 3 : 1) void fwd_dense_kernel(FwdArgs a) {
  using F = DenseForm<W>;
  constexpr int kDRing = F::kRing;
  __shared__ __attribute__((aligned(16))) u16 lds_k[kDRing][kDUE];
  __shared__ __attribute__((aligned(16))) u16 lds_v[kDRing][kDUE];

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, r32 = lane & 31;
  const int g4 = g * 4;  // accumulator element i of lane half g is row acc_row(i, 0) + g4
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // Consecutive workgroups take the key splits of one query tile, then the
  // next tile of the same head, and are dealt to the 8 XCDs round-robin.
  const int logical = blockIdx.x;
  if (logical >= a.total) return;
  const int split = logical % a.splits;
  const int tq = logical / a.splits;
  const int qt = tq % a.n_qt, h = tq / a.n_qt;
  const int row = qt * F::kRows + wave * 32 + r32;
  const bool qvalid = row < a.N;

  QFrag qf;
  load_qfrag(qf, a.q + (int64_t)h * a.N * kHeadDim, row, qvalid, g);
  const u16* kh = a.k + (int64_t)h * a.Nk * kHeadDim;
  const u16* vh = a.v + (int64_t)h * a.Nk * kHeadDim;
  const int Nk = a.Nk;
  const float sl2 = 0.08838834764831845f * kLog2e;  // softmax scale in log2 units

  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
  float l = 0.f;                 // this lane's share of the denominator, relative to 2^m
  float m = -__builtin_inff();   // reference of the running sums (log2 units)

  // The query fragment is the only load the compiler tracks; drain it here so
  // that no wait it places later also waits for the key/value loads below.
  __builtin_amdgcn_s_waitcnt(0);

  // ---- direct loads of one unit (four waves): wave w fills K and V rows 8(w % 4) .. +7 in two
  // groups of four rows (1 KiB per instruction); lane l lands in chunk slot
  // l % 16 of row l / 16 of its group and fetches the global chunk that slot
  // holds.  Offsets are relative to the unit's first key.
  const int slot = lane & 15;
  uint32_t offk[2], offv[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = (wave & 3) * 8 + i * 4 + (lane >> 4);
    offk[i] = (uint32_t)(r * kHeadDim + (kslot(r, slot) << 3)) * 2u;
    offv[i] = (uint32_t)(r * kHeadDim + (vslot(r, slot) << 3)) * 2u;
  }
  // Every unit of the stream starts at a key < Nk (key 0 for the stream past
  // its end); the clamp keeps even a violation of that inside the buffer.
  auto dma_unit = [&](int key0, int st) __attribute__((always_inline)) {
    key0 = min(__builtin_amdgcn_readfirstlane(key0), Nk - 1);
    const u16* kb = kh + (int64_t)key0 * kHeadDim;
    const u16* vb = vh + (int64_t)key0 * kHeadDim;
    if (key0 + kDU <= Nk) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r0 = (wave & 3) * 8 + i * 4;
        dma16_sv(kb, offk[i], lds_addr(&lds_k[st][r0 * kHeadDim]));
        dma16_sv(vb, offv[i], lds_addr(&lds_v[st][r0 * kHeadDim]));
      }
    } else {
      // ragged last unit: rows past the last key re-read the last key (finite
      // data); their scores are masked and their probabilities are zero
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r0 = (wave & 3) * 8 + i * 4;
        const int r = r0 + (lane >> 4);
        const int rr = min(r, Nk - 1 - key0);
        const uint32_t ok = (uint32_t)(rr * kHeadDim + (kslot(r, slot) << 3)) * 2u;
        const uint32_t ov = (uint32_t)(rr * kHeadDim + (vslot(r, slot) << 3)) * 2u;
        dma16_sv(kb, ok, lds_addr(&lds_k[st][r0 * kHeadDim]));
        dma16_sv(vb, ov, lds_addr(&lds_v[st][r0 * kHeadDim]));
      }
    }
  };

  // ---- LDS operand offsets (bytes within a stage), formed once: the K
  // operand of k-step ks, and the V^T operand of 32-dim tile dt (k-step h2 and
  // the second 8 rows add immediates).
  uint32_t kofs[8], vofs[4];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) kofs[ks] = (uint32_t)(r32 * kHeadDim + (kslot(r32, ks * 2 + g) << 3)) * 2u;
  {
    const int G = lane >> 4, j = lane & 15, r0 = g * 4 + (j >> 2);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int col = dt * 32 + (G & 1) * 16 + 4 * (j & 3);
      vofs[dt] = (uint32_t)(r0 * kHeadDim + (vslot(r0, col >> 3) << 3) + (col & 7)) * 2u;
    }
  }
  auto kop = [&](int st, int ks) __attribute__((always_inline)) {
    return *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(&lds_k[st][0]) + kofs[ks]);
  };

  // ---- S^T = K Q^T of one staged unit, the K operands read four at a time
  auto mma_s = [&](int st) __attribute__((always_inline)) {
    f32x16 s = {};
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      u32x4 kf[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kf[ks] = kop(st, b * 4 + ks);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) s = mfma32(as_bf16x8(kf[ks]), qf.k[b * 4 + ks], s);
      __builtin_amdgcn_sched_barrier(0);
    }
    return s;
  };

  // ---- online softmax of one unit's S tile.  Keys past the end are masked
  // first.  `probs` forms the probabilities against the reference as the bf16
  // B operand of the PV product (keys permuted within 16 as the accumulator
  // layout holds them) and returns their row sum, taken over the fp32 values
  // before rounding: the denominator of both the output and lse.  `rebase`,
  // taken only when the probabilities against the current reference overran
  // it (always on a row's first unit, whose reference is -inf), moves the
  // reference to the row maximum, with o and l rescaled.
  auto mask_ragged = [&](f32x16& s, int key0) __attribute__((always_inline)) {
    if (key0 + kDU > Nk) {  // ragged last unit: keys past the end do not exist
      const int lim = Nk - key0;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (g4 >= lim - acc_row(i, 0)) s[i] = -__builtin_inff();
    }
  };
  auto probs = [&](const f32x16& s, bf16x8 (&pb)[2]) __attribute__((always_inline)) -> float {
    const float neg_ref = -m;
    float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float e = fast_exp2(__builtin_fmaf(s[i], sl2, neg_ref));
      pb[i >> 3][i & 7] = (__bf16)e;
      if (i & 8) rs1 += e; else rs0 += e;
    }
    return rs0 + rs1;
  };
  auto rebase = [&](const f32x16& s) __attribute__((always_inline)) {
    float mx = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
    mx = fmaxf(mx, partner_f(mx, g));
    const float mc = mx * sl2;
    const bool up = mc > m;
    if (__ballot(up)) {
      const float alpha = up ? fast_exp2(m - mc) : 1.f;  // 0 on a row's first unit
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
    }
    if (up) m = mc;
  };

  // ---- O^T += V^T P^T: the V^T operand of k-step h2 holds keys
  // h2*16 + {4g..4g+3, 8+4g..8+4g+3} -- the keys of P this lane half holds --
  // read as two transposed 4 x 16 blocks per 16-lane group.
  auto mma_pv = [&](int st, const bf16x8 (&pb)[2]) __attribute__((always_inline)) {
    const char* vst = reinterpret_cast<const char*>(&lds_v[st][0]);
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const char* p = vst + vofs[dt] + h2 * 16 * kHeadDim * 2;
        const u32x2 v0 = lds_read_tr16(reinterpret_cast<const u16*>(p));
        const u32x2 v1 = lds_read_tr16(reinterpret_cast<const u16*>(p + 8 * kHeadDim * 2));
        const u32x4 va = {v0[0], v0[1], v1[0], v1[1]};
        o[dt] = mfma32(as_bf16x8(va), pb[h2], o[dt]);
      }
    }
  };

  // ---- unit stream of this workgroup's key range, and the unit in each
  // stage: its first key, and bit st of `sval` when it holds a unit
  const int t_begin = split * a.tiles_per_split;
  const int t_end = min(a.nb, t_begin + a.tiles_per_split);
  int u_next = t_begin * (kDTile / kDU);
  const int u_end = min(t_end * (kDTile / kDU), (Nk + kDU - 1) / kDU);
  int skey[kDRing];
#pragma unroll
  for (int i = 0; i < kDRing; ++i) skey[i] = 0;
  uint32_t sval = 0;

  // Issues the next unit of the stream into stage st (a stream past its end
  // reloads key 0 into a stage nobody reads, so the count of loads in flight
  // stays exact).
  auto issue_next = [&](const int st, const int grp) __attribute__((always_inline)) {
    const bool have = u_next < u_end;
    const int key0 = have ? u_next * kDU : 0;
    if (have) ++u_next;
    if (W == 4 || (wave >> 2) == grp) dma_unit(key0, st);
    skey[st] = key0;
    sval = have ? (sval | (1u << st)) : (sval & ~(1u << st));
  };

  // The unit in stage st, if it holds one.
  auto compute = [&](const int st) __attribute__((always_inline)) {
    if ((sval >> st) & 1u) {
      f32x16 s = mma_s(st);
      mask_ragged(s, skey[st]);
      bf16x8 pb[2];
      float rsum = probs(s, pb);
      if (__ballot(!(rsum <= kDSlackSum))) {
        rebase(s);
        rsum = probs(s, pb);
      }
      l += rsum;
      mma_pv(st, pb);
    }
  };
  // One iteration for the P units in stages st .. st + P - 1: the units 2P
  // ahead are issued into the stages the previous iteration computed (free
  // since the barrier that ended it).  Returns false once the stream is
  // exhausted and no issued unit is left.
  auto iteration = [&](const int st) __attribute__((always_inline)) -> bool {
#pragma unroll
    for (int j = 0; j < F::P; ++j) issue_next((st + 2 * F::P + j) % kDRing, j);
#pragma unroll
    for (int j = 0; j < F::P; ++j) compute(st + j);
    __builtin_amdgcn_s_waitcnt(F::kWait);  // this wave's loads of the next P units landed
    wg_barrier();                          // ... and every wave's
    bool left = u_next < u_end;
#pragma unroll
    for (int j = F::P; j < kDRing; ++j) left = left || ((sval >> ((st + j) % kDRing)) & 1u) != 0;
    return left;
  };

  // prologue: units 0 .. 2P - 1 into the first 2P stages
#pragma unroll
  for (int j = 0; j < 2 * F::P; ++j) issue_next(j, j % F::P);
  __builtin_amdgcn_s_waitcnt(F::kWait);
  wg_barrier();
  // the loop is unrolled over one turn of the ring, so that every stage index
  // (and with it every LDS offset and load destination) is a constant
  while (iteration(0) && iteration(F::P) && iteration(2 * F::P)) {
  }
  __builtin_amdgcn_s_waitcnt(0);  // no load may land after the workgroup ends

  // ---- epilogue ----
  const float lt = l + partner_f(l, g);
  if (!qvalid) return;
  if (a.splits == 1 && !a.part_o) {
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

hipError_t launch_forward_dense(const FwdArgs& a, hipStream_t s) {
  // Without a key split and with enough 384-row tiles to fill the chip, the
  // W = 12 form; otherwise the W = 4 form on the 128-row tiles of the plan.
  const int n_wide = (a.N + DenseForm<12>::kRows - 1) / DenseForm<12>::kRows;
  if (a.splits == 1 && (long long)a.H * n_wide >= kDWideMinWGs) {
    FwdArgs w = a;
    w.n_qt = n_wide;
    w.total = a.H * n_wide;
    return launch_kernel(fwd_dense_kernel<12>, dim3((w.total + 7) & ~7), dim3(768), s, w);
  }
  const int grid = (a.total + 7) & ~7;
  return launch_kernel(fwd_dense_kernel<4>, dim3(grid), dim3(256), s, a);
}

}  // namespace solattn

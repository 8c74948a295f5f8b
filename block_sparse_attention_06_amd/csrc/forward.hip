// Fused sparse attention forward for gfx950 with a pipelined key loop:
// query-thresholded block-sparse attention with a first-order Taylor term for
// the rejected blocks, in one online-softmax pass.  Dense attention runs in
// fwd_dense_kernel (forward_dense.hip).
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
// four stages filled by direct global->LDS loads.  A load takes a scalar base
// (the unit's first key) and a per-lane offset fixed for the whole kernel, so
// issuing a unit costs no vector arithmetic; the main loop is unrolled over
// one turn of the ring, so stage offsets are immediates in every LDS access.
// (The dense kernel's form -- three workgroups per CU, no software pipeline --
// runs this method's 4K workload in 13 % fewer cycles, but its 96 co-resident
// tiles per XCD no longer sweep the keys in step: 3.5x the fabric traffic,
// L2 hits 54 % instead of 87 %, and the power-limited clock drops by as much.)
//
// Per iteration each wave (1) runs the online softmax of the oldest unit in
// flight on its S tile, computed one iteration earlier, (2) routes and issues
// the loads of the newest unit, (3) issues the S^T = K Q^T products of the next
// unit, and (4) issues O^T += V^T P^T for the oldest unit.  The softmax therefore never
// waits for its own products, and the matrix products of (3) and (4) run while
// the wave crosses the barrier and starts the next softmax.  Each wave then
// waits only for its own loads of the unit whose S comes next, and one barrier
// per unit publishes them and frees the stage refilled next.
#include "device.hpp"
#include "launch.hpp"

namespace solattn {

namespace {

constexpr int kU = 32;                  // keys per staged unit
constexpr int kUE = kU * kHeadDim;      // bf16 per tensor per stage
constexpr int kRing = 4;                // LDS stages (64 KiB: two workgroups per CU)
constexpr int kAhead = kRing - 1;       // units in flight beyond the one whose PV runs
constexpr int kDmaPerUnit = 4;          // loads per wave per unit: 2 groups of 4 rows, K and V
// The running sums' reference may lag a row's maximum by up to 8 (log2
// units): a lane's row sum of one unit's probabilities stays within 2^8.
constexpr float kSlackSum = 256.f;
constexpr int kLgkm0 = 0xC07F;          // s_waitcnt lgkmcnt(0)

// s_waitcnt immediate (gfx9 encoding) for vmcnt(n) alone.
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }
// At the end of an iteration the loads of the next two units (S next, PV
// after) must have landed; the kAhead - 2 younger units may still be in flight.
constexpr int kWaitNext = vmcnt_imm(kDmaPerUnit * (kAhead - 2));

}  // namespace

template <int KB>
__global__ __launch_bounds__(256, 2) void fwd_kernel(FwdArgs a) {
  __shared__ __attribute__((aligned(16))) u16 lds_k[kRing][kUE];
  __shared__ __attribute__((aligned(16))) u16 lds_v[kRing][kUE];

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, r32 = lane & 31;
  const int g4 = g * 4;  // accumulator element i of lane half g is row acc_row(i, 0) + g4
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // Consecutive workgroups take query tiles of one head and are dealt to the
  // 8 XCDs round-robin, so all XCDs work on the same one or two heads at a
  // time; within a head either in natural order or, for a sparse call without
  // a key split, in the order of decreasing work (a.order).
  const int logical = blockIdx.x;
  if (logical >= a.total) return;
  const int split = logical % a.splits;
  const int tq = a.order ? a.order[logical] : logical / a.splits;
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
  float mu = 0.f, tau = __builtin_inff();
  if (qvalid) {
    mu = gload<float>(a.mu + (int64_t)h * a.N + row);
    tau = make_tau(mu, gload<float>(a.sigma + (int64_t)h * a.N + row), a.beta);
  }
  // reference of the running sums (log2 units), within 8 of the max; the
  // Taylor terms are relative to e^mu, so it starts there
  float m = mu * kLog2e;

  // The query fragment and row statistics are the only loads the compiler
  // tracks; drain them here so that no wait it places later also waits for
  // the key/value loads below (which it does not track).
  __builtin_amdgcn_s_waitcnt(0);

  // ---- direct loads of one unit: wave w fills K and V rows 8w .. 8w+7 in two
  // groups of four rows (1 KiB per instruction); lane l lands in chunk slot
  // l % 16 of row l / 16 of its group and fetches the global chunk that slot
  // holds.  Offsets are relative to the unit's first key.
  const int slot = lane & 15;
  uint32_t offk[2], offv[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = wave * 8 + i * 4 + (lane >> 4);
    offk[i] = (uint32_t)(r * kHeadDim + (kslot(r, slot) << 3)) * 2u;
    offv[i] = (uint32_t)(r * kHeadDim + (vslot(r, slot) << 3)) * 2u;
  }
  // Every unit of the stream starts at a key < Nk (key 0 for the stream past
  // its end); the clamp below keeps even a violation of that inside the buffer.
  auto dma_unit = [&](int key0, int st) __attribute__((always_inline)) {
    key0 = min(__builtin_amdgcn_readfirstlane(key0), Nk - 1);
    st = __builtin_amdgcn_readfirstlane(st);
    const u16* kb = kh + (int64_t)key0 * kHeadDim;
    const u16* vb = vh + (int64_t)key0 * kHeadDim;
    if (key0 + kU <= Nk) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r0 = wave * 8 + i * 4;
        dma16_sv(kb, offk[i], lds_addr(&lds_k[st][r0 * kHeadDim]));
        dma16_sv(vb, offv[i], lds_addr(&lds_v[st][r0 * kHeadDim]));
      }
    } else {
      // ragged last unit: rows past the last key re-read the last key (finite
      // data); their scores are masked and their probabilities are zero
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r0 = wave * 8 + i * 4;
        const int r = r0 + (lane >> 4);
        const int rr = min(r, Nk - 1 - key0);
        const uint32_t ok = (uint32_t)(rr * kHeadDim + (kslot(r, slot) << 3)) * 2u;
        const uint32_t ov = (uint32_t)(rr * kHeadDim + (vslot(r, slot) << 3)) * 2u;
        dma16_sv(kb, ok, lds_addr(&lds_k[st][r0 * kHeadDim]));
        dma16_sv(vb, ov, lds_addr(&lds_v[st][r0 * kHeadDim]));
      }
    }
  };

  // ---- S^T = K Q^T of one staged unit (consumed an iteration later): operand
  // reads and products separately, so the products can be interleaved with
  // other work.
  // Byte offsets, within a stage, of this lane's K operand of each k-step and
  // of its V^T operand of each 32-dim tile (k-step h2 and the second 8 rows
  // add constants): formed once, so that each operand read is one register
  // plus an immediate (the stage offsets are compile-time in the unrolled loop).
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
  auto read_k = [&](int st, u32x4 (&kf)[8]) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) kf[ks] = kop(st, ks);
  };
  auto mfma_s = [&](const u32x4 (&kf)[8]) __attribute__((always_inline)) {
    f32x16 s = {};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) s = mfma32(as_bf16x8(kf[ks]), qf.k[ks], s);
    return s;
  };

  // ---- online softmax of one unit's S tile.  Keys past the end are masked
  // first.  The tail forms the probabilities as the bf16 B operand of the PV
  // product (keys permuted within 16 as the accumulator layout holds them)
  // and returns their row sum, taken over the fp32 values before rounding:
  // that sum is the denominator of both the output and lse (a sum of the
  // rounded values would carry their rounding into lse unaveraged where a few
  // keys hold the mass).  The head, taken only when the probabilities
  // against the current reference overran it, finds the row max and moves
  // the reference (m, with o and l rescaled); it returns the exponent offset
  // (-m, or -inf for rows that did not select the unit: p = 0).
  auto mask_ragged = [&](f32x16& s, int key0) __attribute__((always_inline)) {
    if (key0 + kU > Nk) {  // ragged last unit: keys past the end do not exist
      // element i holds key offset acc_row(i, 0) + 4g: compare the one
      // per-lane term with scalar limits (no per-element lane offsets kept live)
      const int lim = Nk - key0;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (g4 >= lim - acc_row(i, 0)) s[i] = -__builtin_inff();
    }
  };
  auto softmax_head = [&](f32x16& s, int key0, bool mine) __attribute__((always_inline)) {
    mask_ragged(s, key0);
    float mx = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
    mx = fmaxf(mx, partner_f(mx, g));
    const float mc = mx * sl2;
    // each selected row's reference moves up to its maximum
    const bool up = mine && (mc > m);
    if (__ballot(up)) {
      const float alpha = up ? fast_exp2(m - mc) : 1.f;
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
    }
    if (up) m = mc;
    return mine ? -m : -__builtin_inff();
  };
  auto softmax_tail = [&](const f32x16& s, float neg_ref, bf16x8 (&pb)[2]) __attribute__((always_inline)) -> float {
    float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float e = fast_exp2(__builtin_fmaf(s[i], sl2, neg_ref));
      pb[i >> 3][i & 7] = (__bf16)e;
      if (i & 8) rs1 += e; else rs0 += e;
    }
    return rs0 + rs1;
  };

  // ---- the softmax tail of one unit interleaved with the S products of the
  // next: product k, then the probabilities of elements 2k and 2k+1 (scale,
  // exponential, bf16 pair, fp32 row sum), fenced so that the compiler keeps
  // the order; K operand reads run four products ahead.
  auto tail_and_s = [&](const f32x16& s_in, float neg_ref, bf16x8 (&pb)[2], int st, float& rsum) __attribute__((always_inline)) {
    u32x4 kf[8];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) kf[ks] = kop(st, ks);
    f32x16 s = {};
    float rs[2] = {0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (k < 4) kf[k + 4] = kop(st, k + 4);
      s = mfma32(as_bf16x8(kf[k]), qf.k[k], s);
      __builtin_amdgcn_sched_barrier(0);
      const float e0 = fast_exp2(__builtin_fmaf(s_in[2 * k], sl2, neg_ref));
      const float e1 = fast_exp2(__builtin_fmaf(s_in[2 * k + 1], sl2, neg_ref));
      pb[k >> 2][(2 * k) & 7] = (__bf16)e0;
      pb[k >> 2][(2 * k + 1) & 7] = (__bf16)e1;
      rs[k >> 2] += e0 + e1;
      __builtin_amdgcn_sched_barrier(0);
    }
    rsum = rs[0] + rs[1];
    return s;
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
        const char* a = vst + vofs[dt] + h2 * 16 * kHeadDim * 2;
        const u32x2 v0 = lds_read_tr16(reinterpret_cast<const u16*>(a));
        const u32x2 v1 = lds_read_tr16(reinterpret_cast<const u16*>(a + 8 * kHeadDim * 2));
        const u32x4 va = {v0[0], v0[1], v1[0], v1[1]};
        o[dt] = mfma32(as_bf16x8(va), pb[h2], o[dt]);
      }
    }
  };

  // ---- unit queue.  Before the shift of iteration i, slot j holds unit
  // i - 1 - kAhead + j and sits in stage (st_issue + j) mod kRing: slot 1 gets
  // its softmax and PV in this iteration (its S tile was computed one
  // iteration earlier), slot 2 its S; the unit issued now enters slot kAhead.
  // Validity / need are wave-uniform bit masks, "mine" (this row selected the
  // unit's block) a per-lane bit mask; bit j = slot j.
  int qkey[kAhead + 1];
#pragma unroll
  for (int i = 0; i <= kAhead; ++i) qkey[i] = 0;
  uint32_t qneed = 0, qval = 0, qmine = 0;
  bool stream_done = false;

  // unit sources: chunks of blocks routed, their selected blocks pending
  int c_next = t_begin, cA = 0;
  uint32_t UA = 0, fullA = 0, wvA = 0;
  int pend_left = 0, pend_key = 0;
  bool pend_mine = false, pend_need = false;
  const u16* khi = a.khi + (int64_t)h * a.nb_pad * kHeadDim;
  const u16* klo = a.klo + (int64_t)h * a.nb_pad * kHeadDim;
  const u16* vsum = a.vsumT + (int64_t)h * kHeadDim * a.nb_pad;

  // One iteration.  s_in holds the S tile of slot 1, s_out receives that of
  // slot 2; the loop below alternates the two tiles so that neither is copied.
  // Returns false once the stream is exhausted and every unit is through its PV.
  auto iteration = [&](f32x16& s_in, f32x16& s_out, const int st_issue) __attribute__((always_inline)) -> bool {
    const int st1 = st_issue == kRing - 1 ? 0 : st_issue + 1;
    const int st2 = st1 == kRing - 1 ? 0 : st1 + 1;
    const bool pv = (qneed & 2u) != 0, do_s = (qneed & 4u) != 0;
    bf16x8 pb[2];
    float neg_ref = 0.f, rsum = 0.f;
    const bool mine1 = (qmine & 2u) != 0;
    // The reference is checked after the fact: the probabilities are formed
    // against it and the unit goes on only if every lane's row sum stays
    // within kSlackSum (which bounds each probability).  A dense row's first
    // unit always fails the check (its reference is still -inf) and sets it.
    if (pv) {
      mask_ragged(s_in, qkey[1]);
      neg_ref = mine1 ? -m : -__builtin_inff();
    }
    // The product-issuing part of the iteration runs at raised wave priority:
    // when both waves of a SIMD are ready, the one feeding the matrix core
    // issues first, and the other's bookkeeping fills the gaps.
    __builtin_amdgcn_s_setprio(1);
    if (pv && do_s) {
      // The probabilities of slot 1 and the S products of slot 2 do not
      // depend on each other: interleave about six vector instructions after
      // each product so that they issue while it runs.
      s_out = tail_and_s(s_in, neg_ref, pb, st2, rsum);
    } else if (pv) {
      rsum = softmax_tail(s_in, neg_ref, pb);
      asm volatile("" : "=v"(s_out));  // unused: defined without an instruction
    } else if (do_s) {
      u32x4 kf[8];
      read_k(st2, kf);
      s_out = mfma_s(kf);
    } else {
      asm volatile("" : "=v"(s_out));  // unused: defined without an instruction
    }
    // Rare after a row's first unit: a row outran the reference.  Move each
    // selected row's reference to its maximum (o and l rescaled) and form the
    // probabilities again.
    if (pv && __ballot(!(rsum <= kSlackSum))) {
      neg_ref = softmax_head(s_in, qkey[1], mine1);
      rsum = softmax_tail(s_in, neg_ref, pb);
    }
    l += rsum;
    if (pv) mma_pv(st1, pb);
    __builtin_amdgcn_s_setprio(0);

      // -- next unit of the stream --
      bool have = false;
      int key0 = 0;
      bool mi = false, ne = false;
      if (!stream_done) {
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
            uint32_t sel_bits = 0;  // this row's selections
            // Weights enter the MFMA as bf16 hi + lo parts: when many blocks
            // share nearly the same weight, a single bf16 rounding would bias
            // the Taylor mass coherently instead of averaging out.
            bf16x8 whi[2], wlo[2];
            float wden = 0.f;
            // element i is block c0 + acc_row(i, 0) + 4g: limits are scalar,
            // the lane term enters through g4 and one shift at the end
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int ci = acc_row(i, 0);
              const bool inr = qvalid && g4 < t_end - c0 - ci;
              const bool sel = inr && is_selected(p[i], tau);
              sel_bits |= (uint32_t)sel << ci;
              const float wt = (inr && !sel) ? (1.f + p[i] - mu) * f : 0.f;
              __bf16 wh, wl;
              split_bf16(wt, wh, wl);
              whi[i >> 3][i & 7] = wh;
              wlo[i >> 3][i & 7] = wl;
              // valid keys of the block (wt = 0 outside the range)
              const int nj = max(0, min(KB, Nk - (c0 + ci) * KB - g4 * KB));
              wden = __builtin_fmaf((float)nj, wt, wden);
            }
            sel_bits <<= g4;
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
            fullA = sel_bits | partner_b(sel_bits, g);
            const uint32_t w = wave_or(sel_bits);  // the wave's selections
            wvA = w;
            // Exchange the wave masks through the last bytes of the K tile of
            // the stage about to be refilled: nothing reads that stage until
            // the unit issued next lands, and the second barrier keeps every
            // read of the masks ahead of that refill.
            uint32_t* wmask = reinterpret_cast<uint32_t*>(&lds_k[st_issue][kUE - 8]);
            if (lane == 0) wmask[wave] = w;
            __builtin_amdgcn_s_waitcnt(kLgkm0);
            wg_barrier();
            uint32_t un = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) un |= wmask[i];
            UA = __builtin_amdgcn_readfirstlane(un);
            __builtin_amdgcn_s_waitcnt(kLgkm0);
            wg_barrier();
            cA = c0;
            c_next += kChunk;
          }
          if (UA) {
            const int b = __builtin_ctz(UA);
            UA &= UA - 1;
            pend_key = (cA + b) * KB;
            // units of the block that hold at least one key (the last block
            // may be ragged)
            pend_left = min(KB / kU, (Nk - pend_key + kU - 1) / kU);
            pend_mine = ((fullA >> b) & 1u) != 0;
            pend_need = ((wvA >> b) & 1u) != 0;
          }
        }
        if (pend_left > 0) {
          have = true;
          key0 = pend_key;
          mi = pend_mine;
          ne = pend_need;
          pend_key += kU;
          --pend_left;
        }
        stream_done = !have;
      }

    // -- issue the newest unit (a stream past its end reloads key 0 into a
    // stage nobody reads, so the count of loads in flight stays exact) --
    dma_unit(key0, st_issue);
#pragma unroll
    for (int i = 0; i < kAhead; ++i) qkey[i] = qkey[i + 1];
    qkey[kAhead] = key0;
    qval = (qval >> 1) | ((uint32_t)have << kAhead);
    qneed = (qneed >> 1) | ((uint32_t)(have && ne) << kAhead);
    qmine = (qmine >> 1) | ((uint32_t)(have && mi) << kAhead);
    __builtin_amdgcn_s_waitcnt(kWaitNext);  // this wave's loads of the next two units landed
    wg_barrier();                           // ... and every wave's
    // done when the stream is exhausted and no issued unit awaits its PV
    return !(stream_done && (qval >> 1) == 0);
  };
  f32x16 sA = {}, sB = {};
  // Iteration i refills stage i mod kRing (slot 1's stage becomes slot 0
  // after the shift); the loop is unrolled over one turn of the ring so that
  // every stage index, and with it every LDS address offset and every load's
  // LDS destination, is a compile-time constant.
  static_assert(kRing == 4, "the loop below is one turn of a four-stage ring");
  while (iteration(sA, sB, 0) && iteration(sB, sA, 1) && iteration(sA, sB, 2) && iteration(sB, sA, 3)) {
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

hipError_t launch_forward(const FwdArgs& a, int B, hipStream_t s) {
  const int grid = (a.total + 7) & ~7;
  if (B == 64) return launch_kernel(fwd_kernel<64>, dim3(grid), dim3(256), s, a);
  return launch_kernel(fwd_kernel<128>, dim3(grid), dim3(256), s, a);
}

}  // namespace solattn

// Long-sequence dense forward kernel for gfx950: plain softmax attention (the
// dense mode of the forward entry point, and its sparse mode with beta = -inf),
// scheduled so that matrix and vector work overlap.  The sparse method runs in
// fwd_kernel, whose independent 4-wave workgroups suit per-wave skipping.
//
// Schedule.  A workgroup is 8 waves on 256 query rows of one head: group 0
// (waves 0-3) owns query rows 0-127, group 1 (waves 4-7) rows 128-255; each
// wave owns 32 rows.  Keys stream through LDS in units of 64 rows of K and V,
// in a ring of four stages filled by direct global->LDS loads two units ahead.
// Per unit u each wave runs phase A -- S^T = K Q^T for unit u and
// O^T += V^T P^T for unit u-1, all MFMA -- and phase B -- the online softmax of
// S(u), all VALU.  The two groups run opposite phases between two barriers
// per unit: while group 0 does A(u), group 1 does B(u-1); then group 0 does
// B(u) while group 1 does A(u).  The two waves sharing a SIMD therefore
// always present one MFMA stream and one VALU stream.
#include <type_traits>

#include "device.hpp"
#include "launch.hpp"

namespace solattn {

namespace {

constexpr int kPPUnit = 64;                          // keys per staged unit
constexpr int kPPStages = 4;                         // LDS ring
constexpr int kPPStageElems = kPPUnit * kHeadDim;    // bf16 per tensor per stage
constexpr float kPPSlackSum = 256.f;                 // 2^8: bound on a lane's row sum of one unit
constexpr int kPPWaitNext = 0x0F74;                  // s_waitcnt vmcnt(4): next unit landed
constexpr int kPPWaitLgkm0 = 0xC07F;                 // s_waitcnt lgkmcnt(0)

// barrier that also pins the compiler's schedule on both sides
__device__ __forceinline__ void pp_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

}  // namespace

__global__ __launch_bounds__(512, 2) void fwd_pp_kernel(FwdArgs a) {
  __shared__ __attribute__((aligned(16))) u16 lds_k[kPPStages][kPPStageElems];
  __shared__ __attribute__((aligned(16))) u16 lds_v[kPPStages][kPPStageElems];

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, r32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;  // 0: phase A first, 1: phase B first

  // natural order: consecutive workgroups take consecutive 256-row tiles of a
  // head, dealt round-robin to the XCDs; all XCDs share one or two heads
  const int logical = blockIdx.x;
  if (logical >= a.total) return;
  const int n_pairs = (a.N + 255) / 256;
  const int tp = logical % n_pairs, h = logical / n_pairs;
  const int row = tp * 256 + wave * 32 + r32;
  const bool qvalid = row < a.N;

  QFrag qf;
  load_qfrag(qf, a.q + (int64_t)h * a.N * kHeadDim, row, qvalid, g);
  const u16* kh = a.k + (int64_t)h * a.Nk * kHeadDim;
  const u16* vh = a.v + (int64_t)h * a.Nk * kHeadDim;
  const int Nk = a.Nk;
  const float sl2 = 0.08838834764831845f * kLog2e;

  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
  float l = 0.f;
  float m = -__builtin_inff();

  // The query fragment and row statistics are the only loads the compiler
  // tracks; drain them here so that no wait it places later also waits for
  // the key/value prefetches below (which it does not track).
  __builtin_amdgcn_s_waitcnt(0);

  // direct global->LDS loads of a unit: wave w fills K and V rows 8w..8w+7,
  // four rows (1 KiB) per instruction; rows past the last key re-read it
  auto dma_unit = [&](int key0, int st) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r0 = wave * 8 + i * 4;
      const int r = r0 + (lane >> 4), slot = lane & 15;
      const int64_t key = min(key0 + r, Nk - 1);
      dma_to_lds16(kh + key * kHeadDim + (kslot(r, slot) << 3), lds_addr(&lds_k[st][r0 * kHeadDim]));
      dma_to_lds16(vh + key * kHeadDim + (vslot(r, slot) << 3), lds_addr(&lds_v[st][r0 * kHeadDim]));
    }
  };

  // unit slots: 0 = unit u-1, 1 = unit u, 2 = unit u+1, 3 = unit u+2
  int qkey[4];
  bool qmine[4], qneed[4], qval[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    qkey[i] = 0;
    qmine[i] = qneed[i] = qval[i] = false;
  }
  f32x16 s[2];
  s[0] = s[1] = f32x16{};
  float o_scale = 1.f;     // pending rescale of o (set by phase B, applied by phase A)
  bool o_rescale = false;  // wave-uniform
  bf16x8 pb[4];
  // V^T operands of the first two products of the next PV step, read at the
  // end of the softmax phase of the same unit (its stage stays resident until
  // that PV step has run)
  constexpr int kVPre = 2;
  u32x4 vpre[kVPre];
#pragma unroll
  for (int i = 0; i < 4; ++i) pb[i] = bf16x8{};

  // ---- unit sources ----
  bool stream_done = false;
  int u_next = 0;
  const int u_end = (Nk + kPPUnit - 1) / kPPUnit;

  auto gen = [&](int& key0, bool& mi, bool& ne) __attribute__((always_inline)) -> bool {
    if (stream_done) return false;
    bool have = false;
    if (u_next < u_end) {
      have = true;
      key0 = u_next * kPPUnit;
      mi = ne = true;
      ++u_next;
    }
    stream_done = !have;
    return have;
  };

  // ---- LDS operand addresses (bytes within a stage), formed per read ----
  // K operand of k-step ks, rows kt*32 + r32: chunk (2ks + g) ^ (r32 % 16);
  // the kt offset is an immediate.
  // V^T operand for d-tile dt: lane j of 16-lane group G reads row
  // (g*4 + j/4) + {kt*32 + h2*16 + 8a}, columns dt*32 + (G%2)*16 + 4(j%4) .. +4;
  // with the V swizzle the chunk is ((dt ^ (j/4 % 4)) * 4 + (G%2)*2 + (j%4)/2).
  const int G = lane >> 4, j = lane & 15;
  const int krow = r32 * 256, kx = g ^ (r32 & 15);
  const int vrow = (g * 4 + (j >> 2)) * 256 + (((G & 1) * 2 + ((j & 3) >> 1)) << 4) + ((j & 1) << 3);
  const int vx = (j >> 2) & 3;
  auto kaddr = [&](int ks) __attribute__((always_inline)) { return krow + (((ks * 2) ^ kx) << 4); };
  auto vaddr = [&](int dt) __attribute__((always_inline)) { return vrow + ((dt ^ vx) << 6); };
  const char* lds_k_bytes = reinterpret_cast<const char*>(&lds_k[0][0]);
  const char* lds_v_bytes = reinterpret_cast<const char*>(&lds_v[0][0]);
  constexpr int kStageBytes = kPPStageElems * 2;

  // ---- phase A: S^T = K Q^T for slot 1, then O^T += V^T P^T for slot 0 ----
  // (the S products first: the softmax after the next barrier waits only for
  // them, while the PV products' tail overlaps it; 0.5 % faster than the
  // other order, same results)
  auto phase_a = [&](int st_prev, int st_cur) __attribute__((always_inline)) {
    if (o_rescale) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[dt] *= o_scale;
      o_scale = 1.f;
      o_rescale = false;
    }
    if (qval[1] && qneed[1]) {
      const char* kst = lds_k_bytes + st_cur * kStageBytes;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        s[kt] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          const u32x4 ka = *reinterpret_cast<const u32x4*>(kst + kaddr(ks) + kt * 32 * 256);
          s[kt] = mfma32(as_bf16x8(ka), qf.k[ks], s[kt]);
        }
      }
    }
    if (qval[0] && qneed[0]) {
      const char* vst = lds_v_bytes + st_prev * kStageBytes;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int roff = (kt * 32 + h2 * 16) * 256;
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) {
            u32x4 va;
            if (kt == 0 && h2 == 0 && dt < kVPre) {
              va = vpre[dt];
            } else {
              const u32x2 v0 = lds_read_tr16(reinterpret_cast<const u16*>(vst + vaddr(dt) + roff));
              const u32x2 v1 = lds_read_tr16(reinterpret_cast<const u16*>(vst + vaddr(dt) + roff + 8 * 256));
              va = u32x4{v0[0], v0[1], v1[0], v1[1]};
            }
            o[dt] = mfma32(as_bf16x8(va), pb[kt * 2 + h2], o[dt]);
          }
        }
      }
    }
  };

  // ---- phase B: online softmax of the scores in s (unit slot `su`) ----
  // The probabilities are formed against the current reference first; the
  // unit goes on only if every lane's row sum stays within kPPSlackSum (which
  // bounds each probability).  Otherwise -- always on a row's first unit,
  // whose reference is still -inf, and rarely after -- each selected row's
  // reference moves to its maximum (the accumulator is rescaled by phase A,
  // before it adds this unit) and the probabilities are formed again.  The
  // row sum is taken over the fp32 probabilities before their rounding to
  // bf16; it is the denominator of the output and of lse.
  auto probs = [&](float neg_ref) __attribute__((always_inline)) -> float {
    float rsum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = fast_exp2(__builtin_fmaf(s[kt][i], sl2, neg_ref));
        pb[kt * 2 + (i >> 3)][i & 7] = (__bf16)e;
        rsum[i & 3] = (kt == 0 && i < 4) ? e : rsum[i & 3] + e;  // first term: no +0
      }
    return (rsum[0] + rsum[1]) + (rsum[2] + rsum[3]);
  };
  auto phase_b = [&](int key0, bool mine, bool need, int st) __attribute__((always_inline)) {
    if (!need) return;
    if (key0 + kPPUnit > Nk) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (key0 + kt * 32 + acc_row(i, g) >= Nk) s[kt][i] = -__builtin_inff();
    }
    float rs = probs(mine ? -m : -__builtin_inff());
    if (__ballot(!(rs <= kPPSlackSum))) {
      float mx = fmaxf(s[0][0], s[1][0]);
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, fmaxf(s[0][i], s[1][i]));
      mx = fmaxf(mx, partner_f(mx, g));
      const float mc = mx * sl2;
      const bool up = mine && (mc > m);
      const float alpha = up ? fast_exp2(m - mc) : 1.f;  // 0 on a row's first unit
      l *= alpha;
      o_scale *= alpha;
      o_rescale = true;
      if (up) m = mc;
      rs = probs(mine ? -m : -__builtin_inff());
    }
    l += rs;
    const char* vst = lds_v_bytes + st * kStageBytes;
#pragma unroll
    for (int dt = 0; dt < kVPre; ++dt) {
      const u32x2 v0 = lds_read_tr16(reinterpret_cast<const u16*>(vst + vaddr(dt)));
      const u32x2 v1 = lds_read_tr16(reinterpret_cast<const u16*>(vst + vaddr(dt) + 8 * 256));
      vpre[dt] = u32x4{v0[0], v0[1], v1[0], v1[1]};
    }
  };

  // ---- prologue: units 0 and 1 into stages 0 and 1 ----
  {
    int k0 = 0, k1 = 0;
    bool m0 = false, n0 = false, m1 = false, n1 = false;
    const bool h0 = gen(k0, m0, n0);
    const bool h1 = h0 && gen(k1, m1, n1);
    qkey[2] = k0; qmine[2] = m0; qneed[2] = n0; qval[2] = h0;
    qkey[3] = k1; qmine[3] = m1; qneed[3] = n1; qval[3] = h1;
    dma_unit(k0, 0);
    dma_unit(k1, 1);
    __builtin_amdgcn_s_waitcnt(kPPWaitNext);
    pp_barrier();
  }

  // The two groups run the same sequence of barriers; only the order of the
  // phases inside a unit differs, so each group gets its own copy of the loop
  // with the order fixed at compile time.
  auto main_loop = [&](auto group) __attribute__((always_inline)) {
    constexpr int GRP = decltype(group)::value;
    for (int u = 0;; ++u) {
      // shift: slot 1 becomes unit u
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        qkey[i] = qkey[i + 1];
        qmine[i] = qmine[i + 1];
        qneed[i] = qneed[i + 1];
        qval[i] = qval[i + 1];
      }
      if (!qval[0] && !qval[1]) break;
      {
        int k3 = 0;
        bool m3 = false, n3 = false;
        const bool h3 = gen(k3, m3, n3);
        qkey[3] = k3; qmine[3] = m3; qneed[3] = n3; qval[3] = h3;
        dma_unit(k3, (u + 2) & 3);  // stage of unit u-2, free since the last barrier
      }
      const int st_prev = (u + 3) & 3, st_cur = u & 3;
      if constexpr (GRP == 0) {
        phase_a(st_prev, st_cur);
        pp_barrier();
        phase_b(qkey[1], qmine[1], qval[1] && qneed[1], st_cur);  // softmax of unit u
      } else {
        phase_b(qkey[0], qmine[0], qval[0] && qneed[0], st_prev);  // softmax of unit u-1
        pp_barrier();
        phase_a(st_prev, st_cur);
      }
      __builtin_amdgcn_s_waitcnt(kPPWaitNext);  // unit u+1 landed
      pp_barrier();
    }
  };
  if (grp == 0)
    main_loop(std::integral_constant<int, 0>{});
  else
    main_loop(std::integral_constant<int, 1>{});
  __builtin_amdgcn_s_waitcnt(0);  // no load may land after the workgroup ends

  // ---- epilogue ----
  const float lt = l + partner_f(l, g);
  if (!qvalid) return;
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
}

hipError_t launch_forward_pp(const FwdArgs& a, hipStream_t s) {
  return launch_kernel(fwd_pp_kernel, dim3(a.total), dim3(512), s, a);
}

}  // namespace solattn

// 3D neighbourhood attention over a video token grid for gfx950.
//
// [DAI] "LTX-2.5 at 4K, in half the time" (doubleAI), section "Inside the
// decoder": the diffusion video decoder spends most of its time in one
// neighbourhood-attention kernel over tiles of four frames.  Each query at
// (t, y, x) attends to the kt x ky x kx keys of a window centred on it and
// shifted inward at the grid's borders (start = clamp(p - k/2, 0, L - k) per
// axis); plain softmax attention with scale 1/sqrt(d) inside the window.
//
// Workgroup: 4 waves on one patch of 4 rows x 8 columns of queries in four
// consecutive frames; wave w owns the patch in frame 4 b + w (32 queries,
// lane l % 32 = one query, in the transposed "lane owns a row" MFMA
// formulation of the attention kernels).  All four waves see the same rows
// and columns of keys (at most 3 + ky rows and 7 + kx columns), and frame
// windows of neighbouring frames overlap, so a key region is loaded once for
// the four frames.  Keys stream through LDS as units of 32 keys -- UR rows of
// UC consecutive columns of one frame (2 x 16 when the patch's columns fit in
// 16, else 1 x 32) -- in a ring of kNRing stages filled by direct global->LDS
// loads kNRing - 1 units ahead (the unit loop is unrolled over one turn of the
// ring, so stage offsets are immediates).  A wave skips the products of units outside
// its frame window; inside a unit, keys outside a query's window get
// probability 0.
#include "device.hpp"
#include "launch.hpp"

namespace solattn {

namespace {

constexpr int kNU = 32;                  // keys per unit
constexpr int kNUE = kNU * kHeadDim;     // bf16 per tensor per stage
constexpr int kNRing = 4;
constexpr int kNAhead = kNRing - 1;      // units in flight ahead of the one computed
constexpr int kNDma = 4;                 // loads per wave per unit (K and V, 2 x 4 keys each)
// vmcnt((kNAhead - 1) * kNDma): all of this wave's loads but those of the
// kNAhead - 1 newest units have landed
constexpr int kNWait = (((kNAhead - 1) * kNDma) & 15) | 0x0F70;
static_assert((kNAhead - 1) * kNDma < 16, "vmcnt field");
constexpr int kPR = 4, kPC = 8;          // query patch: rows x columns

__device__ __forceinline__ int win_start(int p, int len, int k) { return min(max(p - (k >> 1), 0), len - k); }

constexpr float kSlackSum = 256.f;  // 2^8: the reference may lag the row maximum by 8 (log2 units)

}  // namespace

template <int UR>
__global__ __launch_bounds__(256, 2) void na3d_kernel(Na3dArgs a) {
  constexpr int UC = kNU / UR;  // columns per unit row
  __shared__ __attribute__((aligned(16))) u16 lds_k[kNRing][kNUE];
  __shared__ __attribute__((aligned(16))) u16 lds_v[kNRing][kNUE];

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, r32 = lane & 31;
  const int g4 = g * 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int T = a.T, Y = a.Y, X = a.X;

  // Workgroup -> (head, frame group, patch).  Workgroups are dealt to the
  // eight XCDs in turn; when their count allows, the order is remapped so
  // that each XCD runs a contiguous range of patches (neighbours share keys
  // through that XCD's L2).
  const int px_n = (X + kPC - 1) / kPC, py_n = (Y + kPR - 1) / kPR, pt_n = (T + 3) >> 2;
  const int total = px_n * py_n * pt_n * a.H;
  int b = blockIdx.x;
  if ((total & 7) == 0) b = (b & 7) * (total >> 3) + (b >> 3);
  const int px = b % px_n;
  b /= px_n;
  const int py = b % py_n;
  b /= py_n;
  const int pt = b % pt_n;
  const int h = b / pt_n;
  const int x0 = px * kPC, y0 = py * kPR, f0 = pt * 4;

  // this lane's query
  const int fq = f0 + wave, yq = y0 + (r32 >> 3), xq = x0 + (r32 & 7);
  const bool wvalid = fq < T;  // wave-uniform
  const bool qvalid = wvalid && yq < Y && xq < X;
  const int64_t plane = (int64_t)Y * X;
  const int fqc = min(fq, T - 1), yqc = min(yq, Y - 1), xqc = min(xq, X - 1);
  const int64_t qrow = (int64_t)fqc * plane + (int64_t)yqc * X + xqc;
  const int64_t head = (int64_t)h * T * plane * kHeadDim;
  QFrag qf;
  {
    const u32x4* p = reinterpret_cast<const u32x4*>(a.q + head + qrow * kHeadDim);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (qvalid) x = gload<u32x4>(p + ks * 2 + g);
      qf.k[ks] = as_bf16x8(x);
    }
  }
  // window of this lane's query
  const int wy = win_start(yqc, Y, a.ky), wx = win_start(xqc, X, a.kx);
  // frames of this wave's window (wave-uniform)
  const int wf = win_start(fqc, T, a.kt);
  // key region of the workgroup: frames [fa, fb), rows [ya, yb), columns from xu
  const int fa = win_start(f0, T, a.kt);
  const int fb = win_start(min(f0 + 3, T - 1), T, a.kt) + a.kt;
  const int ya = win_start(y0, Y, a.ky);
  const int yb = win_start(min(y0 + kPR - 1, Y - 1), Y, a.ky) + a.ky;
  const int xa = win_start(x0, X, a.kx);
  const int xu = max(0, min(xa, X - UC));  // first column of every unit
  const int nunits = (fb - fa) * ((yb - ya + UR - 1) / UR);

  const char* kh = reinterpret_cast<const char*>(a.k + head);
  const char* vh = reinterpret_cast<const char*>(a.v + head);
  __builtin_amdgcn_s_waitcnt(0);

  // Direct loads of a unit: wave w fills keys 8w .. 8w+7 (two groups of 4,
  // K and V).  Key r of a unit is (row group start + r / UC, xu + r % UC); a
  // lane's byte offset from the unit's first key is fixed for the whole
  // kernel, so a unit costs only its scalar base.  Columns past the grid are
  // clamped to the last one (never inside a window); the row group is moved
  // up so that it ends inside the grid, and its rows before the nominal start
  // are masked (they belong to the previous group).
  const int slot = lane & 15;
  uint32_t koff[2], voff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = wave * 8 + i * 4 + (lane >> 4);
    const uint32_t key = (uint32_t)((r / UC) * X + min(xu + r % UC, X - 1));
    koff[i] = key * (kHeadDim * 2) + (kslot(r, slot) << 4);
    voff[i] = key * (kHeadDim * 2) + (vslot(r, slot) << 4);
  }
  const int ylast = Y - UR;  // last start of a row group that stays in the grid
  auto dma_unit = [&](int ff, int yy, int st) __attribute__((always_inline)) {
    const int64_t base = ((int64_t)ff * plane + (int64_t)min(yy, ylast) * X) * (kHeadDim * 2);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r0 = wave * 8 + i * 4;
      dma16_sv(kh + base, koff[i], lds_addr(&lds_k[st][r0 * kHeadDim]));
      dma16_sv(vh + base, voff[i], lds_addr(&lds_v[st][r0 * kHeadDim]));
    }
  };

  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
  // Running sums relative to a reference m (log2 units) that may lag the row
  // maximum by up to 8: o and l are rescaled only when the maximum outruns it.  The
  // denominator l sums the fp32 exponentials before their rounding to bf16 (with
  // windows of a few dozen keys a sum of the rounded values would carry their
  // rounding into lse unaveraged); it normalises the output and gives lse.  m
  // starts at a finite -1e30, so that a unit without keys of this query
  // (maximum -inf) leaves it alone and its probabilities come out 0.
  float l = 0.f, m = -1e30f;
  const float sl2 = 0.08838834764831845f * kLog2e;
  // column mask of element i (key column xu + acc_row(i, 0) % UC + 4g), as an
  // additive 0 / -inf bias fixed for the kernel; elements i and i + 16 / UR
  // share a column
  constexpr int NC = 16 / UR;
  float cbias[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = xu + acc_row(i, 0) % UC + g4;
    cbias[i] = (c >= wx && c < wx + a.kx) ? 0.f : -__builtin_inff();
  }

  // unit counters (frame, nominal row-group start) of the loads and of the
  // products, advanced without divisions
  int lf = fa, ly = ya, cf = fa, cy = ya;
  auto advance = [&](int& f, int& y) __attribute__((always_inline)) {
    y += UR;
    if (y >= yb) { y = ya; ++f; }
  };
#pragma unroll
  for (int i = 0; i < kNAhead; ++i) {
    dma_unit(min(lf, fb - 1), lf < fb ? ly : yb - 1, i);
    advance(lf, ly);
  }
  // Byte offsets, within a stage, of this lane's K operand of each k-step and
  // of its V^T operand of each 32-dim tile (k-step h2 and the second 8 rows
  // add constants), formed once.
  uint32_t nkofs[8], nvofs[4];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) nkofs[ks] = (uint32_t)(r32 * kHeadDim + (kslot(r32, ks * 2 + g) << 3)) * 2u;
  {
    const int G = lane >> 4, j = lane & 15, r0 = g * 4 + (j >> 2);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int col = dt * 32 + (G & 1) * 16 + 4 * (j & 3);
      nvofs[dt] = (uint32_t)(r0 * kHeadDim + (vslot(r0, col >> 3) << 3) + (col & 7)) * 2u;
    }
  }
  // One unit; st = u mod kNRing.  The loop below is unrolled over one turn of
  // the ring, so st is a compile-time constant in each copy and every LDS
  // access and load destination takes an immediate stage offset.
  auto unit_step = [&](const int u, const int st) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(kNWait);  // this wave's loads of unit u landed
    __builtin_amdgcn_s_barrier();        // ... and every wave's; unit u - 1's stage is free
    asm volatile("" ::: "memory");
    // past the end: re-loads the last unit into a stage that is never read
    dma_unit(min(lf, fb - 1), lf < fb ? ly : yb - 1, (u + kNAhead) % kNRing);
    advance(lf, ly);
    const int ff = cf, ynom = cy;
    advance(cf, cy);
    if (!wvalid || ff < wf || ff >= wf + a.kt) return;  // wave-uniform
    const int yy = min(ynom, ylast);

    // S^T = K Q^T for the unit's 32 keys
    f32x16 s = {};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const u32x4 kf = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(&lds_k[st][0]) + nkofs[ks]);
      s = mfma32(as_bf16x8(kf), qf.k[ks], s);
    }
    // rows of the unit inside this query's window (and not before the group's
    // nominal start); columns outside it carry the -inf column bias
    const int rlo = max(wy, ynom), rhi = wy + a.ky;
    float rbias[UR];
#pragma unroll
    for (int rr = 0; rr < UR; ++rr) rbias[rr] = (yy + rr >= rlo && yy + rr < rhi) ? 0.f : -__builtin_inff();
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] += cbias[i % NC];
    // Probabilities against the current reference first; the unit goes on
    // only if the lane's row sum stays within kSlackSum (which bounds each
    // probability).  Otherwise -- a query's first unit with keys in its window
    // (the reference is still -1e30: the sums overflow), or rarely a query that
    // outran it -- the row maxima move the reference and the probabilities
    // are formed again.
    bf16x8 pb[2];
    float rs = 0.f;
    auto probs = [&]() __attribute__((always_inline)) {
      float nref[UR];
#pragma unroll
      for (int rr = 0; rr < UR; ++rr) nref[rr] = rbias[rr] - m;
      rs = 0.f;
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const float e0 = fast_exp2(__builtin_fmaf(s[i], sl2, nref[acc_row(i, 0) / UC]));
        const float e1 = fast_exp2(__builtin_fmaf(s[i + 1], sl2, nref[acc_row(i + 1, 0) / UC]));
        pb[i >> 3][i & 7] = (__bf16)e0;
        pb[i >> 3][(i & 7) + 1] = (__bf16)e1;
        rs += e0 + e1;
      }
    };
    probs();
    if (__ballot(!(rs <= kSlackSum))) {
      float mxr[UR];
#pragma unroll
      for (int rr = 0; rr < UR; ++rr) mxr[rr] = -__builtin_inff();
#pragma unroll
      for (int i = 0; i < 16; ++i) mxr[acc_row(i, 0) / UC] = fmaxf(mxr[acc_row(i, 0) / UC], s[i]);
      float mx = -__builtin_inff();
#pragma unroll
      for (int rr = 0; rr < UR; ++rr) mx = fmaxf(mx, mxr[rr] + rbias[rr]);
      // partner lane l ^ 32 holds the other 16 keys of the same query
      const float mc = pair_max(mx) * sl2;
      const bool up = mc > m;
      const float alpha = up ? fast_exp2(m - mc) : 1.f;
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
      if (up) m = mc;
      probs();
    }
    l += rs;
    // O^T += V^T P^T (as in the attention kernels: two transposing reads per
    // 16-key half and 32-dim tile)
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const char* va = reinterpret_cast<const char*>(&lds_v[st][0]) + nvofs[dt] + h2 * 16 * kHeadDim * 2;
        const u32x2 v0 = lds_read_tr16(reinterpret_cast<const u16*>(va));
        const u32x2 v1 = lds_read_tr16(reinterpret_cast<const u16*>(va + 8 * kHeadDim * 2));
        o[dt] = mfma32(as_bf16x8(u32x4{v0[0], v0[1], v1[0], v1[1]}), pb[h2], o[dt]);
      }
    }
    };
  static_assert(kNRing == 4, "the loop below is one turn of a four-stage ring");
  for (int u = 0; u < nunits; u += kNRing) {
    unit_step(u, 0);
    if (u + 1 < nunits) unit_step(u + 1, 1);
    if (u + 2 < nunits) unit_step(u + 2, 2);
    if (u + 3 < nunits) unit_step(u + 3, 3);
  }
  __builtin_amdgcn_s_waitcnt(0);  // no load may land after the workgroup ends

  // epilogue: the query's denominator is split over lanes l and l ^ 32
  const float lt = pair_sum(l);
  if (!qvalid) return;
  const float inv = 1.f / lt;
  u16* orow = a.out + head + qrow * kHeadDim;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int b4 = 0; b4 < 4; ++b4) {
      const int d0 = dt * 32 + b4 * 8 + g4;
      u32x2 pk;
      pk[0] = (uint32_t)f32_to_bf16_bits(o[dt][4 * b4] * inv) | ((uint32_t)f32_to_bf16_bits(o[dt][4 * b4 + 1] * inv) << 16);
      pk[1] = (uint32_t)f32_to_bf16_bits(o[dt][4 * b4 + 2] * inv) | ((uint32_t)f32_to_bf16_bits(o[dt][4 * b4 + 3] * inv) << 16);
      *reinterpret_cast<u32x2*>(orow + d0) = pk;
    }
  if (a.lse && g == 0) a.lse[(int64_t)h * T * plane + qrow] = m * kLn2 + logf(lt);
}

hipError_t launch_na3d(const Na3dArgs& a, hipStream_t s) {
  const int wgs = ((a.X + kPC - 1) / kPC) * ((a.Y + kPR - 1) / kPR) * ((a.T + 3) / 4) * a.H;
  // the patch's key columns (at most kPC - 1 + kx) fit in a 16-column unit
  // row (and the grid has the two rows of a unit)
  if (kPC - 1 + a.kx <= 16 && a.Y >= 2) return launch_kernel(na3d_kernel<2>, dim3(wgs), dim3(256), s, a);
  return launch_kernel(na3d_kernel<1>, dim3(wgs), dim3(256), s, a);
}

}  // namespace solattn

// 3D neighbourhood attention over a video token grid for gfx950.
//
// [DAI] "LTX-2.5 at 4K, in half the time" (doubleAI), section "Inside the
// decoder": the diffusion video decoder spends most of its time in one
// neighbourhood-attention kernel over tiles of four frames.  Each query at
// (t, y, x) attends to the kt x ky x kx keys of a window centred on it and
// shifted inward at the grid's borders (start = clamp(p - k/2, 0, L - k) per
// axis); plain softmax attention with scale 1/sqrt(d) inside the window.
//
// Workgroup: 4 waves on a brick of 1 frame x 8 rows x 16 columns of queries;
// wave w owns rows 2w and 2w + 1 (32 queries, lane l % 32 = one query, in the
// transposed "lane owns a row" MFMA formulation of the attention kernels).
// The keys any query of the brick can see are kt frames x (8 + ky - 1) rows x
// at most 16 + kx - 1 <= 32 columns; they stream through LDS as units of one
// (frame, row) and 32 consecutive columns (K and V, 16 KiB), in a
// three-stage ring filled by direct global->LDS loads two units ahead.  A wave
// skips the products of units whose row no query of it can see; inside a
// unit, keys outside a query's window get probability 0.
#include "device.hpp"
#include "launch.hpp"

namespace solattn {

namespace {

constexpr int kNU = 32;                  // keys per unit (one row segment)
constexpr int kNUE = kNU * kHeadDim;     // bf16 per tensor per stage
constexpr int kNRing = 3;
constexpr int kNDma = 4;                 // loads per wave per unit (K and V, 2 x 4 rows each)
constexpr int kNWaitNext = (kNDma & 15) | 0x0F70;  // vmcnt(4): the next unit landed

__device__ __forceinline__ int n_kslot(int row, int c) { return c ^ (row & 15); }
__device__ __forceinline__ int n_vslot(int row, int c) { return c ^ ((row & 3) << 2); }

__device__ __forceinline__ int win_start(int p, int len, int k) { return min(max(p - (k >> 1), 0), len - k); }

}  // namespace

__global__ __launch_bounds__(256, 2) void na3d_kernel(Na3dArgs a) {
  __shared__ __attribute__((aligned(16))) u16 lds_k[kNRing][kNUE];
  __shared__ __attribute__((aligned(16))) u16 lds_v[kNRing][kNUE];

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, r32 = lane & 31;
  const int g4 = g * 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int T = a.T, Y = a.Y, X = a.X;

  // brick: consecutive workgroups take neighbouring column bricks of a row band
  const int bx_n = (X + 15) >> 4, by_n = (Y + 7) >> 3;
  int b = blockIdx.x;
  const int bx = b % bx_n;
  b /= bx_n;
  const int by = b % by_n;
  const int t = b / by_n;
  const int h = blockIdx.y;
  const int x0 = bx * 16, y0 = by * 8;

  // this lane's query
  const int yq = y0 + 2 * wave + (r32 >> 4), xq = x0 + (r32 & 15);
  const bool qvalid = yq < Y && xq < X;
  const int64_t plane = (int64_t)Y * X;
  const int64_t qrow = (int64_t)t * plane + (int64_t)min(yq, Y - 1) * X + min(xq, X - 1);
  const u16* qh = a.q + (int64_t)h * T * plane * kHeadDim;
  QFrag qf;
  {
    const u32x4* p = reinterpret_cast<const u32x4*>(qh + qrow * kHeadDim);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (qvalid) x = gload<u32x4>(p + ks * 2 + g);
      qf.k[ks] = as_bf16x8(x);
    }
  }
  // window of this lane's query (rows and columns; the frames of the brick's
  // units are exactly the frame window)
  const int wy = win_start(min(yq, Y - 1), Y, a.ky), wx = win_start(min(xq, X - 1), X, a.kx);
  // rows any query of this wave sees (wave-uniform)
  const int wy_lo = win_start(min(y0 + 2 * wave, Y - 1), Y, a.ky);
  const int wy_hi = win_start(min(y0 + 2 * wave + 1, Y - 1), Y, a.ky) + a.ky;
  // units of the brick
  const int ts = win_start(t, T, a.kt);
  const int ya = win_start(y0, Y, a.ky);
  const int yb = win_start(min(y0 + 7, Y - 1), Y, a.ky) + a.ky;  // exclusive
  const int xa = win_start(x0, X, a.kx);
  const int xu = max(0, min(xa, X - kNU));  // first column of every unit
  const int nrows = yb - ya;
  const int nunits = a.kt * nrows;

  const u16* kh = a.k + (int64_t)h * T * plane * kHeadDim;
  const u16* vh = a.v + (int64_t)h * T * plane * kHeadDim;
  __builtin_amdgcn_s_waitcnt(0);

  // direct loads of unit u: wave w fills K and V rows 8w .. 8w+7 (columns
  // xu + row, clamped to the last column: those keys are never in a window)
  const int slot = lane & 15;
  auto dma_unit = [&](int u, int st) __attribute__((always_inline)) {
    u = min(u, nunits - 1);
    const int tt = ts + u / nrows, yy = ya + u % nrows;
    const int64_t base = (int64_t)tt * plane + (int64_t)yy * X;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r0 = wave * 8 + i * 4;
      const int r = r0 + (lane >> 4);
      const int64_t key = base + min(xu + r, X - 1);
      dma_to_lds16(kh + key * kHeadDim + (n_kslot(r, slot) << 3), lds_addr(&lds_k[st][r0 * kHeadDim]));
      dma_to_lds16(vh + key * kHeadDim + (n_vslot(r, slot) << 3), lds_addr(&lds_v[st][r0 * kHeadDim]));
    }
  };

  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
  // two denominators: of the bf16 probabilities the PV product uses (the
  // output's normaliser, so weights sum to one exactly as multiplied) and of
  // the fp32 exponentials (for lse: with windows of a few dozen keys the bf16
  // rounding of p would not average out)
  float l = 0.f, l32 = 0.f, m = -__builtin_inff();
  const float sl2 = 0.08838834764831845f * kLog2e;

  dma_unit(0, 0);
  dma_unit(1, 1);
  for (int u = 0; u < nunits; ++u) {
    const int st = u % kNRing;
    __builtin_amdgcn_s_waitcnt(kNWaitNext);  // this wave's loads of unit u landed
    __builtin_amdgcn_s_barrier();            // ... and every wave's; unit u - 1's stage is free
    asm volatile("" ::: "memory");
    dma_unit(u + 2, (u + 2) % kNRing);       // past the end: re-loads the last unit (never read)
    const int yy = ya + u % nrows;
    if (yy < wy_lo || yy >= wy_hi) continue;  // wave-uniform: no query of this wave sees the row

    // S^T = K Q^T for the unit's 32 keys
    f32x16 s = {};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const u32x4 kf = *reinterpret_cast<const u32x4*>(&lds_k[st][r32 * kHeadDim + (n_kslot(r32, ks * 2 + g) << 3)]);
      s = mfma32(as_bf16x8(kf), qf.k[ks], s);
    }
    // keys outside this query's window: row test once, column test per key
    // (element i holds key column xu + acc_row(i, 0) + 4g)
    const bool row_in = yy >= wy && yy < wy + a.ky;
    const int lo = wx - xu - g4, hi = wx + a.kx - xu - g4;  // acc_row(i,0) in [lo, hi)
    float mx = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int c = acc_row(i, 0);
      if (!row_in || c < lo || c >= hi) s[i] = -__builtin_inff();
      mx = fmaxf(mx, s[i]);
    }
    // partner lane l ^ 32 holds the other 16 keys of the same query
    const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    mx = fmaxf(__uint_as_float(pr[0]), __uint_as_float(pr[1]));
    const float mn = fmaxf(m, mx * sl2);
    const float base = mn == -__builtin_inff() ? 0.f : mn;
    const bool up = mn > m;
    if (__ballot(up)) {
      const float alpha = fast_exp2(m - base);
      l *= alpha;
      l32 *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
    }
    m = mn;
    bf16x8 pb[2];
    float rs = 0.f, rs32 = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float e = fast_exp2(__builtin_fmaf(s[i], sl2, -base));
      const __bf16 p = (__bf16)e;
      pb[i >> 3][i & 7] = p;
      rs += (float)p;
      rs32 += e;
    }
    l += rs;
    l32 += rs32;
    // O^T += V^T P^T (as in the attention kernels: two transposing reads per
    // 16-key half and 32-dim tile)
    const int G = lane >> 4, j = lane & 15;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int r0 = h2 * 16 + g * 4 + (j >> 2);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const int col = dt * 32 + (G & 1) * 16 + 4 * (j & 3);
        const u32x2 v0 = lds_read_tr16(&lds_v[st][r0 * kHeadDim + (n_vslot(r0, col >> 3) << 3) + (col & 7)]);
        const u32x2 v1 = lds_read_tr16(&lds_v[st][(r0 + 8) * kHeadDim + (n_vslot(r0 + 8, col >> 3) << 3) + (col & 7)]);
        o[dt] = mfma32(as_bf16x8(u32x4{v0[0], v0[1], v1[0], v1[1]}), pb[h2], o[dt]);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // no load may land after the workgroup ends

  // epilogue: the query's denominator is split over lanes l and l ^ 32
  const auto pl = __builtin_amdgcn_permlane32_swap(__float_as_uint(l), __float_as_uint(l), false, false);
  const float lt = __uint_as_float(pl[0]) + __uint_as_float(pl[1]);
  const auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(l32), __float_as_uint(l32), false, false);
  const float lt32 = __uint_as_float(p32[0]) + __uint_as_float(p32[1]);
  if (!qvalid) return;
  const float inv = 1.f / lt;
  u16* orow = a.out + ((int64_t)h * T * plane + qrow) * kHeadDim;
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
  if (a.lse && g == 0) a.lse[(int64_t)h * T * plane + qrow] = m * kLn2 + logf(lt32);
}

hipError_t launch_na3d(const Na3dArgs& a, hipStream_t s) {
  const int bricks = ((a.X + 15) / 16) * ((a.Y + 7) / 8) * a.T;
  na3d_kernel<<<dim3(bricks, a.H), 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace solattn

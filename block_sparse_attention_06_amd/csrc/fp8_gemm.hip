// FP8 projection GEMM for gfx950: activations quantised to E4M3 with one scale
// per row, weights in E4M3 with one scale per output channel, products on the
// FP8 matrix cores with FP32 accumulation, output bf16.
//
// [DAI] "LTX-2.5 at 4K, in half the time" (doubleAI), section "Thinner seams":
// the refinement pass keeps its weights in FP8, converts the activations to FP8
// with a separate scale for each row and accumulates in FP32, so the matrix
// units run at their FP8 rate.
//
//   quantize_rows_kernel:  s_i = amax_i / 448,  q_ik = RNE_e4m3(x_ik * (448 / amax_i))
//   fp8_gemm_kernel:       y_in = s_i * sw_n * sum_k dec(q_ik) dec(w_nk)   (bf16)
//
// v_mfma_f32_32x32x64_f8f6f4 with E4M3 operands (checked on gfx950 with an
// in-bounds probe): lane l supplies row l % 32 of A (column l % 32 of B) with
// 32 of the 64 k values, lane half l / 32 taking bytes [32 (l / 32), +32) of
// the k slice; the accumulator layout is that of the bf16 32x32 MFMA (lane l
// holds column l % 32, rows 8(i/4) + 4(l/32) + i%4).  Both operands are read
// K-contiguous, so neither needs a transpose.
#include "device.hpp"
#include "launch.hpp"

namespace solattn {

namespace {

constexpr float kE4m3Max = 448.f;

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

}  // namespace

// ---------------------------------------------------------------------------
// Row quantisation.  One wave per row, 8 bf16 (16 bytes) per lane per step:
// pass 1 finds the row's absolute maximum, pass 2 scales, clamps to +-448 (a
// scaled maximum may land one float32 ulp above it) and converts pairs with
// v_cvt_pk_fp8_f32 (round to nearest even).  Rows of up to kQuantKeep * 512
// elements stay in registers between the passes, so the row is read once;
// longer rows are read again (from cache) in pass 2.
// ---------------------------------------------------------------------------
constexpr int kQuantKeep = 8;

__device__ __forceinline__ u32x2 quant8(u32x4 v, float inv) {
  u32x2 out;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float f[4];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      f[2 * e] = __uint_as_float(v[2 * h + e] << 16) * inv;
      f[2 * e + 1] = __uint_as_float(v[2 * h + e] & 0xFFFF0000u) * inv;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = fminf(fmaxf(f[e], -kE4m3Max), kE4m3Max);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], w, true);
    out[h] = (uint32_t)w;
  }
  return out;
}

__device__ __forceinline__ float absmax8(u32x4 v, float m) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    m = fmaxf(m, fabsf(__uint_as_float(v[e] << 16)));
    m = fmaxf(m, fabsf(__uint_as_float(v[e] & 0xFFFF0000u)));
  }
  return m;
}

__global__ __launch_bounds__(256) void quantize_rows_kernel(Fp8QuantArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.M) return;
  const u16* x = a.x + row * a.K;
  uint8_t* q = a.q + row * a.K;
  float amax = 0.f;
  if (a.K <= kQuantKeep * 512) {
    u32x4 keep[kQuantKeep];
#pragma unroll
    for (int i = 0; i < kQuantKeep; ++i) {
      const int k = lane * 8 + i * 512;
      keep[i] = k < a.K ? gload_nt<u32x4>(x + k) : u32x4{0u, 0u, 0u, 0u};  // read once
      amax = absmax8(keep[i], amax);
    }
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) amax = fmaxf(amax, __shfl_xor(amax, sh));
    const float inv = amax > 0.f ? kE4m3Max / amax : 0.f;
    if (lane == 0) a.scale[row] = amax / kE4m3Max;
#pragma unroll
    for (int i = 0; i < kQuantKeep; ++i) {
      const int k = lane * 8 + i * 512;
      if (k < a.K) *reinterpret_cast<u32x2*>(q + k) = quant8(keep[i], inv);
    }
    return;
  }
  for (int k = lane * 8; k < a.K; k += 512) amax = absmax8(gload<u32x4>(x + k), amax);
#pragma unroll
  for (int sh = 1; sh < 64; sh <<= 1) amax = fmaxf(amax, __shfl_xor(amax, sh));
  const float inv = amax > 0.f ? kE4m3Max / amax : 0.f;
  if (lane == 0) a.scale[row] = amax / kE4m3Max;
  for (int k = lane * 8; k < a.K; k += 512)
    *reinterpret_cast<u32x2*>(q + k) = quant8(gload<u32x4>(x + k), inv);
}

namespace {

// ---------------------------------------------------------------------------
// GEMM.  Workgroup: 8 waves (two per SIMD) on a 256 (tokens) x 256 (channels)
// output tile; wave (wm, wn) owns 128 tokens x 64 channels as 4 x 2 MFMA tiles
// computed transposed (D = W A^T: lane l holds token l % 32 and, per tile,
// channels in groups of four consecutive ones, so each store writes 8
// contiguous bytes).  K streams through a five-stage LDS ring in slices of 64
// bytes per row (16 KiB of tokens + 16 KiB of weights per stage), filled by
// direct global->LDS loads four slices ahead; while one wave of a SIMD waits
// for its operands the other issues products.  A row's four 16-byte chunks
// sit at chunk c ^ ((row / 4) % 4), so the 16 lanes of each read phase hit 16
// distinct bank groups.
// ---------------------------------------------------------------------------
constexpr int kGT = 256;              // tile edge (tokens and channels)
constexpr int kGK = 64;               // K bytes per stage
constexpr int kGStages = 5;
constexpr int kGStageBytes = kGT * kGK;  // per operand
constexpr int kGWaves = 8;
constexpr int kGDmaPerStage = 4;         // per wave: 2 token + 2 weight instructions

__device__ __forceinline__ int g_chunk(int row, int c) { return c ^ ((row >> 2) & 3); }

__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

}  // namespace

__global__ __launch_bounds__(512, 1) void fp8_gemm_kernel(Fp8GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[kGStages][kGStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t lds_w[kGStages][kGStageBytes];

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, r32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;

  // XCD-aware order: workgroup b runs on XCD b % 8; the tiles of one XCD are
  // consecutive in (token tile, channel tile) order, channel tile fastest, so
  // the channel tiles of one token tile share that XCD's L2.
  const int per_xcd = a.grid / 8;
  const int logical = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (logical >= a.tiles_m * a.tiles_n) return;
  const int tm = logical / a.tiles_n, tn = logical % a.tiles_n;
  const int m0 = tm * kGT, n0 = tn * kGT;
  const int K = a.K;

  // direct loads: instruction i of this wave fills rows 16 (2 wave + i) .. +15
  // of a stage; lane l lands in row + l / 4, chunk slot l % 4
  const uint8_t* abase[2];
  const uint8_t* wbase[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = (wave * 2 + i) * 16 + (lane >> 2);
    const int c = g_chunk(r, lane & 3);
    // rows past the end re-read the last row (finite data, never stored)
    const int ra = min(m0 + r, a.M - 1), rw = min(n0 + r, a.N - 1);
    abase[i] = a.a + (int64_t)ra * K + c * 16;
    wbase[i] = a.w + (int64_t)rw * K + c * 16;
  }
  auto dma_stage = [&](int ks, int st) __attribute__((always_inline)) {
    const int64_t k0 = (int64_t)ks * kGK;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r0 = (wave * 2 + i) * 16;
      dma_to_lds16(abase[i] + k0, lds_addr(&lds_a[st][r0 * kGK]));
      dma_to_lds16(wbase[i] + k0, lds_addr(&lds_w[st][r0 * kGK]));
    }
  };

  // operand reads: 32 bytes of row R (chunks 2g, 2g+1)
  auto frag = [&](const uint8_t* base, int R) __attribute__((always_inline)) {
    const u32x4 lo = *reinterpret_cast<const u32x4*>(base + R * kGK + (g_chunk(R, 2 * g) << 4));
    const u32x4 hi = *reinterpret_cast<const u32x4*>(base + R * kGK + (g_chunk(R, 2 * g + 1) << 4));
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  // Every step issues one slice of loads (past the last slice it re-loads the
  // last slice into the stage just freed, which is never read again), so the
  // loads in flight are the same at every wait and each wait is one fixed
  // instruction.
  const int nk = K / kGK;
  constexpr int kYoung = (kGStages - 2) * kGDmaPerStage;  // loads of younger slices in flight
  constexpr int kWaitSlice = (kYoung & 15) | ((kYoung >> 4) << 14) | 0x0F70;
#pragma unroll
  for (int s = 0; s < kGStages - 1; ++s) dma_stage(min(s, nk - 1), s);
  for (int s = 0; s < nk; ++s) {
    // this wave's loads of slice s landed (younger slices may be in flight)
    __builtin_amdgcn_s_waitcnt(kWaitSlice);
    __builtin_amdgcn_s_barrier();  // every wave: slice s landed, slice s - 1's stage read
    asm volatile("" ::: "memory");
    dma_stage(min(s + kGStages - 1, nk - 1), (s + kGStages - 1) % kGStages);
    const int st = s % kGStages;
    i32x8 am[4], wf[2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) am[mt] = frag(lds_a[st], wm * 128 + mt * 32 + r32);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) wf[nt] = frag(lds_w[st], wn * 64 + nt * 32 + r32);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) acc[mt][nt] = mfma_fp8(wf[nt], am[mt], acc[mt][nt]);
  }
  __builtin_amdgcn_s_waitcnt(0);

  // epilogue: y[m][n] = acc * sa[m] * sw[n] in bf16, staged through LDS so that
  // every store writes whole 128-byte rows.  Each wave owns 16 KiB of the
  // (now idle) ring: its 128 x 64 tile, row-major, 16-byte chunk c of row r at
  // c ^ (r % 8).  Lane l holds token row 32 mt + l % 32 and, per tile, the
  // channels 32 nt + 8 b + 4 g + (0..3).
  __builtin_amdgcn_s_barrier();  // every wave has read its last operands
  asm volatile("" ::: "memory");
  constexpr int kWaveTileBytes = 128 * 64 * 2;  // 128 tokens x 64 channels of bf16
  uint8_t* stage = (wave < 4 ? &lds_a[0][0] : &lds_w[0][0]) + (wave & 3) * kWaveTileBytes;
  float swr[2][4][4];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int n = min(n0 + wn * 64 + nt * 32 + 8 * b + 4 * g, a.N - 4);
      const f32x4v v = gload<f32x4v>(a.sw + n);
#pragma unroll
      for (int e = 0; e < 4; ++e) swr[nt][b][e] = v[e];
    }
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int r = mt * 32 + r32;
    const float sm = a.sa[min(m0 + wm * 128 + r, a.M - 1)];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        u32x2 pk;
        pk[0] = (uint32_t)f32_to_bf16_bits(acc[mt][nt][4 * b] * sm * swr[nt][b][0]) |
                ((uint32_t)f32_to_bf16_bits(acc[mt][nt][4 * b + 1] * sm * swr[nt][b][1]) << 16);
        pk[1] = (uint32_t)f32_to_bf16_bits(acc[mt][nt][4 * b + 2] * sm * swr[nt][b][2]) |
                ((uint32_t)f32_to_bf16_bits(acc[mt][nt][4 * b + 3] * sm * swr[nt][b][3]) << 16);
        const int c = nt * 4 + b;  // 16-byte chunk of the 128-byte row; half g
        *reinterpret_cast<u32x2*>(stage + r * 128 + ((c ^ (r & 7)) << 4) + g * 8) = pk;
      }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // this wave's LDS writes done (wave-private region)
  const int nw = n0 + wn * 64;
  if (nw < a.N) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = i * 8 + (lane >> 3), pc = lane & 7;
      const int m = m0 + wm * 128 + r;
      const u32x4 v = *reinterpret_cast<const u32x4*>(stage + r * 128 + (pc << 4));
      if (m < a.M) *reinterpret_cast<u32x4*>(a.y + (int64_t)m * a.N + nw + ((pc ^ (r & 7)) << 3)) = v;
    }
  }
}

hipError_t launch_quantize_rows(const Fp8QuantArgs& a, hipStream_t s) {
  const int64_t blocks = (a.M + 3) / 4;
  return launch_kernel(quantize_rows_kernel, dim3((unsigned)blocks), dim3(256), s, a);
}

hipError_t launch_fp8_gemm(const Fp8GemmArgs& a0, hipStream_t s) {
  Fp8GemmArgs a = a0;
  a.tiles_m = (a.M + kGT - 1) / kGT;
  a.tiles_n = (a.N + kGT - 1) / kGT;
  a.grid = (a.tiles_m * a.tiles_n + 7) & ~7;
  return launch_kernel(fp8_gemm_kernel, dim3(a.grid), dim3(kGWaves * 64), s, a);
}

}  // namespace solattn

// Exact merges of partial attention answers for gfx950: the N-way combine of
// split-KV partials (unnormalised numerator, running max, denominator) and the
// two-way LSE merge of finished (out, lse) pairs.
//
// doubleAI page, "Attention across two GPUs": partial answers over disjoint key
// ranges, each carrying its log-sum-exp, merge exactly into the full answer.
#include "device.hpp"
#include "launch.hpp"

namespace solattn {

// ---------------------------------------------------------------------------
// Exact N-way merge of split partials (unnormalised numerator, max, denominator).
// 32 threads per (head, row), 4 dimensions each: 16-byte reads of every
// split's numerator, 8-byte bf16 stores, 8 rows per 256-thread workgroup.
// ---------------------------------------------------------------------------
constexpr int kCombineRows = 8;

__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int64_t HN = (int64_t)a.H * a.N;
  const int64_t rg = (int64_t)blockIdx.x * kCombineRows + (threadIdx.x >> 5);  // h * N + row
  if (rg >= HN) return;
  const int d0 = (threadIdx.x & 31) * 4;
  float M = -__builtin_inff();
  for (int s = 0; s < a.splits; ++s) M = fmaxf(M, a.part_ml[(s * HN + rg) * 2]);
  const float mref = M == -__builtin_inff() ? 0.f : M;
  f32x4 num = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  for (int s = 0; s < a.splits; ++s) {
    const float w = exp2f(a.part_ml[(s * HN + rg) * 2] - mref);
    den += w * a.part_ml[(s * HN + rg) * 2 + 1];
    const f32x4 x = *reinterpret_cast<const f32x4*>(a.part_o + (s * HN + rg) * kHeadDim + d0);
#pragma unroll
    for (int e = 0; e < 4; ++e) num[e] += w * x[e];
  }
  u32x2 pk;
  pk[0] = (uint32_t)f32_to_bf16_bits(num[0] / den) | ((uint32_t)f32_to_bf16_bits(num[1] / den) << 16);
  pk[1] = (uint32_t)f32_to_bf16_bits(num[2] / den) | ((uint32_t)f32_to_bf16_bits(num[3] / den) << 16);
  *reinterpret_cast<u32x2*>(a.out + rg * kHeadDim + d0) = pk;
  if (d0 == 0 && a.lse) a.lse[rg] = mref * kLn2 + logf(den);
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  const int64_t rows = (int64_t)a.H * a.N;
  return launch_kernel(combine_kernel, dim3((unsigned)((rows + kCombineRows - 1) / kCombineRows)),
                       dim3(256), s, a);
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
  return launch_kernel(merge_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), s, a);
}

}  // namespace solattn

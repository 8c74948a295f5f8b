// Device-side building blocks shared by the gfx950 kernels of libsolattn.
//
// Wave64 MFMA conventions used throughout (checked on gfx950):
//   v_mfma_f32_32x32x16_bf16, D[32x32] += A[32x16] * B[16x32]:
//     lane l supplies A row (l % 32), k = 8*(l / 32) .. +8 and
//                     B col (l % 32), k = 8*(l / 32) .. +8;
//     lane l holds    D col (l % 32), rows 8*(i/4) + 4*(l/32) + (i%4), i < 16.
// Every attention product is computed transposed (S^T = K Q^T, O^T = V^T P^T),
// so that each lane owns one query row (column l % 32) and all of that row's
// accumulators: row maxima, rescaling and Taylor weights need no shuffles
// beyond one exchange with the partner lane l ^ 32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace solattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16;

constexpr int kHeadDim = 128;
constexpr int kChunk = 32;       // key blocks routed together (one MFMA tile of blocks)
constexpr int kQTile = 128;      // query rows per workgroup (4 waves x 32)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// Loads through the global address space (vector memory counter only; a
// generic pointer would become a flat load, which also holds up LDS waits).
template <class T>
__device__ __forceinline__ T gload(const void* p) {
  typedef const T __attribute__((address_space(1))) global_t;
  return *(global_t*)p;
}

// Load of data a kernel reads once, as a stream: non-temporal, so it does not
// displace reused lines from the caches.  Only for data whose lines one
// instruction uses whole; a layout that touches a line from several
// instructions would lose the line between them.
template <typename T>
__device__ __forceinline__ T gload_nt(const void* p) {
  typedef const T __attribute__((address_space(1))) global_t;
  return __builtin_nontemporal_load((global_t*)p);
}

__device__ __forceinline__ float bf16_to_f32(u16 b) { return __uint_as_float((uint32_t)b << 16); }

// Round to nearest even (finite inputs).
__device__ __forceinline__ u16 f32_to_bf16_bits(float x) {
  return __builtin_bit_cast(u16, (__bf16)x);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Position of block/key k (0..15) inside its group of 16 in the permuted
// "k-major" layouts: lane half g of an MFMA operand reads positions 8g..8g+7,
// which hold keys {4g..4g+3, 8+4g..8+4g+3} -- the keys that lane half holds in
// the accumulator layout above.
__device__ __forceinline__ int perm16(int k) { return ((k & 7) >> 2) * 8 + (k >> 3) * 4 + (k & 3); }

// Offset, inside a 32-wide accumulator tile, of element i held by lane half g.
__device__ __forceinline__ int acc_row(int i, int g) { return (i >> 2) * 8 + g * 4 + (i & 3); }

// Query fragment of one wave: lane l holds row (l % 32) of the wave's 32 rows,
// k-step ks covers dims 16 ks + 8 (l/32) .. +8.
struct QFrag {
  bf16x8 k[8];
};

__device__ __forceinline__ void load_qfrag(QFrag& qf, const u16* qhead, int row, bool valid, int g) {
  const u32x4* p = reinterpret_cast<const u32x4*>(qhead + (int64_t)row * kHeadDim);
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (valid) x = gload<u32x4>(p + ks * 2 + g);
    qf.k[ks] = as_bf16x8(x);
  }
}

// Split of an fp32 value into bf16 hi + lo (both round to nearest even):
// hi + lo carries ~16 significant bits.  Every producer of the bf16 parts of
// the pooled keys uses this one function, so the parts are bit-identical
// wherever they are formed.
__device__ __forceinline__ void split_bf16(float x, __bf16& hi, __bf16& lo) {
  hi = (__bf16)x;
  lo = (__bf16)(x - (float)hi);
}

// Proxy scores p = (q . kbar_j) / sqrt(d) of the wave's 32 rows against the 32
// pooled keys b0 .. b0+31 (Sol-Engine LTX25 page, "Stage 2 Optimization --
// Core Technology: Sol-Attn": block proxy scores from pooled keys).
// kbar enters the bf16 MFMA as hi + lo bf16 parts (q is exact in bf16), so p
// carries ~16 significant bits of kbar instead of 8.  `load(ks, hi, lo)`
// supplies the A operand of k-step ks for block row b0 + (lane % 32).
// Result element i of lane l: block b0 + acc_row(i, l/32), query row l % 32.
// Every kernel that routes runs this same MFMA sequence on bit-identical
// operands, so the proxy scores the inspection exports report are the ones
// the forward kernel compares.
template <class Load>
__device__ __forceinline__ f32x16 proxy_tile(const QFrag& qf, Load load) {
  f32x16 acc = {};
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    // operands in two batches of four k-steps: bounds the registers held by
    // loads in flight inside the forward kernel
    if (ks == 4) __builtin_amdgcn_sched_barrier(0);
    bf16x8 hi, lo;
    load(ks, hi, lo);
    acc = mfma32(hi, qf.k[ks], acc);
    acc = mfma32(lo, qf.k[ks], acc);
  }
  const float scale = 0.08838834764831845f;  // 1/sqrt(128)
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] *= scale;
  return acc;
}

// Proxy tile from fp32 pooled keys in global memory (rows >= nb are clamped;
// callers ignore those elements).
__device__ __forceinline__ f32x16 proxy_chunk(const QFrag& qf, const float* kbar_head, int b0,
                                              int nb, int lane) {
  const int g = lane >> 5;
  int blk = b0 + (lane & 31);
  blk = blk < nb ? blk : nb - 1;
  const f32x4* row = reinterpret_cast<const f32x4*>(kbar_head + (int64_t)blk * kHeadDim);
  return proxy_tile(qf, [&](int ks, bf16x8& hi, bf16x8& lo) __attribute__((always_inline)) {
    const f32x4 x0 = gload<f32x4>(row + ks * 4 + g * 2);
    const f32x4 x1 = gload<f32x4>(row + ks * 4 + g * 2 + 1);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      __bf16 h, l;
      split_bf16(x0[e], h, l);
      hi[e] = h;
      lo[e] = l;
      split_bf16(x1[e], h, l);
      hi[e + 4] = h;
      lo[e + 4] = l;
    }
  });
}

// Proxy tile from the bf16 hi / lo parts of the pooled keys ([nb_pad, 128]
// each, zero rows past nb), as the pool kernel writes them for the forward pass.
__device__ __forceinline__ f32x16 proxy_chunk_hl(const QFrag& qf, const u16* khi_head,
                                                 const u16* klo_head, int b0, int lane) {
  const int g = lane >> 5;
  const int64_t off = (int64_t)(b0 + (lane & 31)) * kHeadDim + g * 8;
  return proxy_tile(qf, [&](int ks, bf16x8& hi, bf16x8& lo) __attribute__((always_inline)) {
    hi = as_bf16x8(gload<u32x4>(khi_head + off + ks * 16));
    lo = as_bf16x8(gload<u32x4>(klo_head + off + ks * 16));
  });
}

// Direct global -> LDS load of 16 bytes per lane: lane l's bytes land at LDS
// byte address lds_base + 16 l (lds_base must be wave-uniform; it goes through
// M0).  Issued through inline assembly on purpose: the compiler then does not
// treat it as a pending write to every LDS location, and does not hold the
// following LDS reads of other buffers until it lands.  The caller orders it
// with explicit vector-memory waits (s_waitcnt vmcnt) and barriers.  The
// compiler warns that M0 is reserved; the generated code of these kernels
// never keeps a value of its own in M0 (every M0 write is one of these
// statements, directly followed by its load: checked on the assembly by a test).
__device__ __forceinline__ void dma_to_lds16(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gptr), "s"(lds_base)
               : "memory", "m0");
}

// Direct global -> LDS load of 16 bytes per lane from sbase + voff (sbase
// wave-uniform, voff a 32-bit per-lane byte offset): one scalar base per
// issue, no vector address arithmetic.  Lane l's bytes land at LDS byte
// address lds + 16 l.  Ordered by the caller's explicit vmcnt waits and
// barriers, as dma_to_lds16.
__device__ __forceinline__ void dma16_sv(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds)
               : "memory", "m0");
}

// LDS layouts of a staged key/value unit ([keys][128 bf16], 16-byte chunks)
// in the attention kernels: K rows put chunk c at c ^ (row % 16), so the S
// operand reads 16 consecutive rows at one chunk without bank conflicts; V
// rows put chunk c at c ^ 4 (row % 4), so the transposing read of 4
// consecutive rows x 4 chunks per 16 lanes is conflict-free.
__device__ __forceinline__ int kslot(int row, int c) { return c ^ (row & 15); }
__device__ __forceinline__ int vslot(int row, int c) { return c ^ ((row & 3) << 2); }

// Value held by the partner lane l ^ 32 (lane half g = l / 32): the two
// halves of a query row's accumulators in the transposed MFMA layout.
__device__ __forceinline__ float partner_f(float x, int g) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(g ? r[0] : r[1]);
}

__device__ __forceinline__ uint32_t partner_b(uint32_t x, int g) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return g ? r[0] : r[1];
}

// OR of a 32-bit value over the 64 lanes of a wave (every lane active), as a
// wave-uniform value: shifts within each row of 16 lanes leave the row's OR in
// its lane 15, two row broadcasts carry rows 0-1 into lane 31 and all four
// rows into lane 63, which is read out.  Lanes without a source take 0.
__device__ __forceinline__ uint32_t wave_or(uint32_t x) {
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

// Sum and maximum over the lane pair (l, l ^ 32); the same value in both lanes.
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Workgroup barrier that is also a compiler barrier for memory accesses (the
// hardware barrier alone does not stop the compiler from moving LDS reads).
__device__ __forceinline__ void wg_barrier() {
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// LDS byte address of a pointer into __shared__ memory.
template <class T>
__device__ __forceinline__ uint32_t lds_addr(const T* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)(const char*)p;
}

// gfx950 transposing LDS read: in each group of 16 lanes, lane j reads 4
// consecutive b16 values at its address; lane i of the group receives value
// (i % 4) of lanes 4e + i/4 for e = 0..3.  With lane j pointing at
// row r0 + j/4, column c0 + 4 (j % 4) of a row-major b16 matrix, lane i gets
// the column c0 + i of rows r0 .. r0+3.
__device__ __forceinline__ u32x2 lds_read_tr16(const u16* p) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)p);
  return __builtin_bit_cast(u32x2, r);
}

// Row threshold tau = mu + beta sigma (Sol-Engine LTX25 page, bullet
// "Query-dependent thresholding").  beta = +inf selects nothing.
__device__ __forceinline__ float make_tau(float mu, float sigma, float beta) {
  if (__builtin_isinf(beta)) return beta > 0.f ? __builtin_inff() : -__builtin_inff();
  return __builtin_fmaf(beta, sigma, mu);
}

// A block is attended exactly when its proxy is at or above the threshold.
__device__ __forceinline__ bool is_selected(float p, float tau) { return p >= tau; }

}  // namespace solattn

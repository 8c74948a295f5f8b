// Internal launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace solattn {

struct PoolArgs {
  const uint16_t* k;
  const uint16_t* v;
  float* kbar;      // [H, nb, 128]
  float* vbar;      // [H, nb, 128]
  // The forward pass's routing forms, written by forms_kernel after the pool
  // when khi is set (khi, klo and vsumT are set together; all null for the
  // pool alone):
  uint16_t* vsumT;  // [H, 128, nb_pad] bf16 block sums, permuted groups of 16
  uint16_t* khi;    // [H, nb_pad, 128] bf16 hi part of kbar (zero rows past nb)
  uint16_t* klo;    // [H, nb_pad, 128] bf16 lo part
  int N, H, B, nb, nb_pad;
};

struct StatsArgs {
  const uint16_t* q;
  const float* kbar;
  float* mu;
  float* sigma;
  int N, H, nb;
};

// Moment form of the row statistics: mbar = mean_j kbar_j and the covariance
// C = mean_j (kbar_j - mbar)(kbar_j - mbar)^T of the pooled keys, per head.
// The pooled keys are split into kMomentSplits ranges of blocks; each range's
// shifted partial sums (128 x 128 second moment, only its blocks on or above
// the diagonal written; 128 row sums, which are also the column sums) go to
// `part` before the final kernel adds them.  The last 128 floats of a range's
// slot are spare.
constexpr int kMomentSplits = 8;
constexpr int kMomentPartFloats = 128 * 128 + 2 * 128;

struct MomentArgs {
  const float* kbar;  // [H, nb, 128]
  uint16_t* chi;      // [H, 128, 128] bf16 hi part of C, rows permuted for the MFMA A operand
  uint16_t* clo;      // [H, 128, 128] bf16 lo part
  float* mbar;        // [H, 128]
  float* part;        // [H, kMomentSplits, kMomentPartFloats] partial sums
  int H, nb;
};

struct StatsMomentArgs {
  const uint16_t* q;
  const uint16_t* chi;
  const uint16_t* clo;
  const float* mbar;
  float* mu;
  float* sigma;
  int N, H;
};

struct Fp8QuantArgs {
  const uint16_t* x;  // [M, K] bf16
  uint8_t* q;         // [M, K] E4M3
  float* scale;       // [M]
  int64_t M;
  int K;
};

struct Fp8GemmArgs {
  const uint8_t* a;   // [M, K] E4M3 activations
  const float* sa;    // [M]
  const uint8_t* w;   // [N, K] E4M3 weights
  const float* sw;    // [N]
  uint16_t* y;        // [M, N] bf16
  int M, N, K;
  int tiles_m, tiles_n, grid;  // set by the launcher
};

struct Na3dArgs {
  const uint16_t* q;  // [H, T*Y*X, 128] bf16, frame-major then row-major
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* out;
  float* lse;         // [H, T*Y*X] or null
  int T, Y, X, H;
  int kt, ky, kx;     // odd window sizes, kx <= 25
};

struct ProxyArgs {
  const uint16_t* q;
  const float* kbar;
  float* p;  // [H, nrows, nb]
  int row0, nrows, N, H, nb;
};

struct MaskArgs {
  const uint16_t* q;
  const float* kbar;
  const float* mu;
  const float* sigma;
  float beta;
  uint8_t* mask;  // [H, nrows, nb] or null
  unsigned long long* counts;  // [4]
  int row0, nrows, N, H, nb;
};

struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* out;
  float* lse;          // may be null
  const uint16_t* khi;  // sparse only: bf16 parts of the pooled keys
  const uint16_t* klo;
  const uint16_t* vsumT;
  const float* mu;
  const float* sigma;
  float* part_o;       // [S, H, N, 128] when S > 1, or a key share's partial (S = 1)
  float* part_ml;      // [S, H, N, 2]   (max in log2 units, denominator)
  float beta;
  int N, Nk, H;
  int nb, nb_pad;      // key tiles (sparse: blocks of B) and padded count
  int n_qt;            // query tiles (32 rows per wave)
  int splits, tiles_per_split;
  int total;           // H * n_qt * splits
  const int* order;    // splits == 1: [H * n_qt] query tile of each workgroup, or null
};

// Order of the query tiles of a sparse call: each tile's work (key blocks any
// of its rows selects) counted, then each head's tiles ranked by it.
struct TileOrderArgs {
  const uint16_t* q;
  const uint16_t* khi;  // routing forms of the pooled keys, as FwdArgs
  const uint16_t* klo;
  const float* mu;
  const float* sigma;
  int* work;            // [H, n_qt] (written)
  int* order;           // [H * n_qt] (written)
  float beta;
  int N, H, nb, nb_pad, n_qt;
};

struct CombineArgs {
  const float* part_o;
  const float* part_ml;
  uint16_t* out;
  float* lse;
  int N, H, splits;
};

struct MergeArgs {
  const uint16_t* out_a;
  const float* lse_a;
  const uint16_t* out_b;
  const float* lse_b;
  uint16_t* out;
  float* lse;
  int N, H;
};

// Launch of a one-argument kernel returning the status of this launch alone:
// hipLaunchKernel reports the error of the launch it makes, where
// hipGetLastError would also return (and clear) an earlier, unrelated error
// of the calling thread.
template <class A>
inline hipError_t launch_kernel(void (*kernel)(A), dim3 grid, dim3 block, hipStream_t s, A arg) {
  void* args[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, args, 0, s);
}

hipError_t launch_pool(const PoolArgs& a, hipStream_t s);
hipError_t launch_stats(const StatsArgs& a, hipStream_t s);
hipError_t launch_moments(const MomentArgs& a, hipStream_t s);
hipError_t launch_stats_moment(const StatsMomentArgs& a, hipStream_t s);
hipError_t launch_proxy(const ProxyArgs& a, hipStream_t s);
hipError_t launch_mask(const MaskArgs& a, hipStream_t s);
hipError_t launch_tile_order(const TileOrderArgs& a, hipStream_t s);
constexpr int kOrderMaxTiles = 4096;  // query tiles per head the rank kernel holds in LDS
hipError_t launch_forward(const FwdArgs& a, int B, hipStream_t s);  // sparse
hipError_t launch_forward_dense(const FwdArgs& a, hipStream_t s);
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);
hipError_t launch_merge(const MergeArgs& a, hipStream_t s);
hipError_t launch_quantize_rows(const Fp8QuantArgs& a, hipStream_t s);
hipError_t launch_fp8_gemm(const Fp8GemmArgs& a, hipStream_t s);
hipError_t launch_na3d(const Na3dArgs& a, hipStream_t s);

}  // namespace solattn

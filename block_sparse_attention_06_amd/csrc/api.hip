// C ABI of libsolattn (declared in include/solattn.h): argument checks,
// workspace layout, split planning and kernel launches on the caller's stream.
// Nothing here allocates, frees or synchronises.
#include <math.h>
#include <mutex>
#include <stddef.h>
#include <stdint.h>

#include "solattn.h"
#include "launch.hpp"

using namespace solattn;

// Device scratch of the allocation-free forward entry point: a file-scope
// array, one copy per GPU the library runs on, held until the process ends.
// Host code never uses the array's name as an address (on the host it is only
// a stand-in for the symbol): the device address of each GPU's copy comes from
// hipGetSymbolAddress with that GPU current, once per device, and is kept.
static constexpr size_t kScratchBytes = size_t(128) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kCUs = 256;            // MI355X compute units
// workgroups wanted when the keys are split: one full round of two per CU
// (a second round costs more in per-workgroup start-up and partials than it
// gains: 126 x 2 x 65,280 cross-attention 0.50 -> 0.43 ms)
constexpr int kSplitTarget = 2 * kCUs;
// From this many key blocks on, the row statistics use the moment form (2 d^2
// multiply-adds per row instead of 2 d nb).
constexpr int kMomentMinBlocks = 128;
// From this many query tiles on (four rounds of two workgroups per CU), a
// sparse call without a key split runs each head's tiles in order of
// decreasing work (tile_work_kernel, tile_order_kernel).
constexpr long long kOrderMinTiles = 4LL * 2 * kCUs;
constexpr size_t kMomentBytesPerHead = 2 * 128 * 128 * sizeof(uint16_t) + 128 * sizeof(float) +
                                       (size_t)kMomentSplits * kMomentPartFloats * sizeof(float);

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
int cdiv(int a, int b) { return (a + b - 1) / b; }

// Whether a launch without a key split runs its query tiles in order of
// decreasing work (enough tiles for several rounds of workgroups, and few
// enough per head for the rank kernel's LDS).
bool orders_tiles(int N, int H) {
  const int n_qt = cdiv(N, 128);
  return (long long)H * n_qt >= kOrderMinTiles && n_qt <= kOrderMaxTiles;
}

struct Split {
  int nb, nb_pad, splits, tiles_per_split;
};

// Short query sets leave most CUs idle (one workgroup per 128 rows per head);
// then the key tiles are split over workgroups (doubleAI page, "Attention
// across two GPUs": split the work along the keys) and merged afterwards.
Split plan_split(int N, int Nk, int H, int KB, bool sparse) {
  Split p{};
  p.nb = cdiv(Nk, KB);
  p.nb_pad = (int)round_up((size_t)p.nb, 32);
  const long long wgs = (long long)H * cdiv(N, 128);
  p.splits = 1;
  p.tiles_per_split = p.nb;
  if (wgs < 2 * kCUs) {
    int target = (int)((kSplitTarget + wgs - 1) / wgs);
    if (target > p.nb) target = p.nb;
    int tps = cdiv(p.nb, target);
    if (sparse) tps = (int)round_up((size_t)tps, 32);  // routing chunks stay aligned
    p.tiles_per_split = tps;
    p.splits = cdiv(p.nb, tps);
  }
  return p;
}

struct Plan {
  Split sp, dn;  // sparse plan (blocks of B) and dense plan (tiles of 128 keys)
  int max_splits;
  size_t off_kbar, off_vbar, off_vsum, off_khi, off_klo, off_mu, off_sigma, off_po, off_pml, bytes;
  size_t off_chi, off_clo, off_mbar, off_mpart;  // moment-form statistics (nb >= kMomentMinBlocks)
  size_t off_work, off_order;                     // tile order (sparse, no key split, many tiles)
  bool moments, order;
};

// Sizes are validated by the caller.  A sparse-mode workspace also covers the
// dense kernel, which runs when beta = -inf.
Plan make_plan(int N, int Nk, int H, int B, int mode) {
  Plan p{};
  const bool sparse = mode == SOL_SPARSE;
  p.dn = plan_split(N, Nk, H, 128, false);
  p.max_splits = p.dn.splits;
  if (sparse) {
    p.sp = plan_split(N, Nk, H, B, true);
    if (p.sp.splits > p.max_splits) p.max_splits = p.sp.splits;
  }
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = round_up(off + bytes, 256);
    return o;
  };
  const size_t HN = (size_t)H * N;
  if (sparse) {
    p.off_kbar = take((size_t)H * p.sp.nb * 128 * sizeof(float));
    p.off_vbar = take((size_t)H * p.sp.nb * 128 * sizeof(float));
    p.off_vsum = take((size_t)H * 128 * p.sp.nb_pad * sizeof(uint16_t));
    p.off_khi = take((size_t)H * p.sp.nb_pad * 128 * sizeof(uint16_t));
    p.off_klo = take((size_t)H * p.sp.nb_pad * 128 * sizeof(uint16_t));
    p.off_mu = take(HN * sizeof(float));
    p.off_sigma = take(HN * sizeof(float));
    p.moments = p.sp.nb >= kMomentMinBlocks;
    if (p.moments) {
      p.off_chi = take((size_t)H * 128 * 128 * sizeof(uint16_t));
      p.off_clo = take((size_t)H * 128 * 128 * sizeof(uint16_t));
      p.off_mbar = take((size_t)H * 128 * sizeof(float));
    p.off_mpart = take((size_t)H * kMomentSplits * kMomentPartFloats * sizeof(float));
    }
    p.order = p.sp.splits == 1 && orders_tiles(N, H);
    if (p.order) {
      p.off_work = take((size_t)H * cdiv(N, 128) * sizeof(int));
      p.off_order = take((size_t)H * cdiv(N, 128) * sizeof(int));
    }
  }
  if (p.max_splits > 1) {
    p.off_po = take((size_t)p.max_splits * HN * 128 * sizeof(float));
    p.off_pml = take((size_t)p.max_splits * HN * 2 * sizeof(float));
  }
  p.bytes = off;
  return p;
}

// Workspace of one key share (sol_attn_forward_shard): the pooled local
// blocks and their routing forms, mu and sigma of every row, and the moment
// buffers when the whole sequence has kMomentMinBlocks blocks or more.  No key
// split inside a share, so no partial buffers.
struct ShardPlan {
  int nb, nb_pad;
  size_t off_kbar, off_vbar, off_vsum, off_khi, off_klo, off_mu, off_sigma;
  size_t off_chi, off_clo, off_mbar, off_mpart, off_work, off_order, bytes;
  bool moments, order;
};

ShardPlan make_shard_plan(int N, int Nk, int nb_all, int H, int B, bool sparse) {
  ShardPlan p{};
  p.nb = cdiv(Nk, sparse ? B : 128);
  p.nb_pad = (int)round_up((size_t)p.nb, 32);
  if (!sparse) return p;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = round_up(off + bytes, 256);
    return o;
  };
  const size_t HN = (size_t)H * N;
  p.off_kbar = take((size_t)H * p.nb * 128 * sizeof(float));
  p.off_vbar = take((size_t)H * p.nb * 128 * sizeof(float));
  p.off_vsum = take((size_t)H * 128 * p.nb_pad * sizeof(uint16_t));
  p.off_khi = take((size_t)H * p.nb_pad * 128 * sizeof(uint16_t));
  p.off_klo = take((size_t)H * p.nb_pad * 128 * sizeof(uint16_t));
  p.off_mu = take(HN * sizeof(float));
  p.off_sigma = take(HN * sizeof(float));
  p.moments = nb_all >= kMomentMinBlocks;
  if (p.moments) {
    p.off_chi = take((size_t)H * 128 * 128 * sizeof(uint16_t));
    p.off_clo = take((size_t)H * 128 * 128 * sizeof(uint16_t));
    p.off_mbar = take((size_t)H * 128 * sizeof(float));
    p.off_mpart = take((size_t)H * kMomentSplits * kMomentPartFloats * sizeof(float));
  }
  // the share's tiles in order of decreasing work over its own blocks
  p.order = orders_tiles(N, H);
  if (p.order) {
    p.off_work = take((size_t)H * cdiv(N, 128) * sizeof(int));
    p.off_order = take((size_t)H * cdiv(N, 128) * sizeof(int));
  }
  p.bytes = off;
  return p;
}

int hip_status(hipError_t e) { return e == hipSuccess ? SOL_OK : SOL_ERR_HIP; }

int check_shape(int N, int H, int d) {
  if (N <= 0 || H <= 0) return SOL_ERR_INVALID_ARG;
  if (d != 128) return SOL_ERR_UNSUPPORTED;
  return SOL_OK;
}

int check_block(int B) { return (B == 64 || B == 128) ? SOL_OK : SOL_ERR_UNSUPPORTED; }

// Argument checks of the forward call (Nk = 0 already replaced by N).
int check_forward(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* out,
                  int N, int H, int d, int B, float beta, int mode, int Nk) {
  if (!q || !k || !v || !out) return SOL_ERR_INVALID_ARG;
  if (Nk < 0) return SOL_ERR_INVALID_ARG;
  if (int r = check_shape(N, H, d)) return r;
  if (mode != SOL_DENSE && mode != SOL_SPARSE) return SOL_ERR_UNSUPPORTED;
  if (mode == SOL_SPARSE) {
    if (int r = check_block(B)) return r;
    if (isnan(beta)) return SOL_ERR_INVALID_ARG;
  }
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
    return SOL_ERR_INVALID_ARG;
  return SOL_OK;
}

// The routing steps of a sparse call on a checked, large enough workspace:
// block means of keys and values with the forward kernel's forms, then the
// row statistics (moment form from kMomentMinBlocks blocks on).
struct Routing {
  PoolArgs pool;
  float* mu;
  float* sigma;
};

int route(const uint16_t* q, const uint16_t* k, const uint16_t* v, int N, int H, int B, int Nk,
          const Plan& p, char* ws, hipStream_t s, Routing* out) {
  const Split& sp = p.sp;
  PoolArgs pa{k, v, (float*)(ws + p.off_kbar), (float*)(ws + p.off_vbar),
              (uint16_t*)(ws + p.off_vsum), (uint16_t*)(ws + p.off_khi),
              (uint16_t*)(ws + p.off_klo), Nk, H, B, sp.nb, sp.nb_pad};
  if (int r = hip_status(launch_pool(pa, s))) return r;
  float* mu = (float*)(ws + p.off_mu);
  float* sigma = (float*)(ws + p.off_sigma);
  if (p.moments) {
    MomentArgs ma{pa.kbar, (uint16_t*)(ws + p.off_chi), (uint16_t*)(ws + p.off_clo),
                  (float*)(ws + p.off_mbar), (float*)(ws + p.off_mpart), H, sp.nb};
    if (int r = hip_status(launch_moments(ma, s))) return r;
    StatsMomentArgs sm{q, ma.chi, ma.clo, ma.mbar, mu, sigma, N, H};
    if (int r = hip_status(launch_stats_moment(sm, s))) return r;
  } else {
    StatsArgs sa{q, pa.kbar, mu, sigma, N, H, sp.nb};
    if (int r = hip_status(launch_stats(sa, s))) return r;
  }
  *out = Routing{pa, mu, sigma};
  return SOL_OK;
}

// Launches of the forward call on a checked, large enough workspace.
int forward_launch(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* out,
                   float* lse, int N, int H, int B, float beta, int mode, int Nk, const Plan& p,
                   void* workspace, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const bool sparse = mode == SOL_SPARSE && !(isinf(beta) && beta < 0);
  const Split& sp = sparse ? p.sp : p.dn;

  FwdArgs f{};
  f.q = q; f.k = k; f.v = v; f.out = out; f.lse = lse;
  f.beta = beta; f.N = N; f.Nk = Nk; f.H = H;
  f.nb = sp.nb; f.nb_pad = sp.nb_pad;
  f.n_qt = cdiv(N, 128);
  f.splits = sp.splits; f.tiles_per_split = sp.tiles_per_split;
  f.total = H * f.n_qt * f.splits;
  if (sparse) {
    Routing rt;
    if (int r = route(q, k, v, N, H, B, Nk, p, ws, s, &rt)) return r;
    f.khi = rt.pool.khi; f.klo = rt.pool.klo; f.vsumT = rt.pool.vsumT;
    f.mu = rt.mu; f.sigma = rt.sigma;
    if (p.order) {
      TileOrderArgs ta{q, rt.pool.khi, rt.pool.klo, rt.mu, rt.sigma, (int*)(ws + p.off_work),
                       (int*)(ws + p.off_order), beta, N, H, sp.nb, sp.nb_pad, f.n_qt};
      if (int r = hip_status(launch_tile_order(ta, s))) return r;
      f.order = ta.order;
    }
  }
  if (f.splits > 1) {
    f.part_o = (float*)(ws + p.off_po);
    f.part_ml = (float*)(ws + p.off_pml);
  }
  if (int r = hip_status(sparse ? launch_forward(f, B, s) : launch_forward_dense(f, s))) return r;
  if (f.splits > 1) {
    CombineArgs c{f.part_o, f.part_ml, out, lse, N, H, f.splits};
    if (int r = hip_status(launch_combine(c, s))) return r;
  }
  return SOL_OK;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch address on the device that runs `stream` (the current device
// for the null stream).
int scratch_of_stream_device(void* stream, void** out) {
  int cur = 0, dev = 0;
  if (hipGetDevice(&cur) != hipSuccess) return SOL_ERR_HIP;
  dev = cur;
  if (stream && hipStreamGetDevice((hipStream_t)stream, &dev) != hipSuccess) return SOL_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return SOL_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return SOL_ERR_HIP;
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return SOL_ERR_HIP;
    if (e != hipSuccess || !ptr) return SOL_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SOL_OK;
}


}  // namespace

extern "C" {

const char* sol_attn_error_string(int code) {
  switch (code) {
    case SOL_OK: return "ok";
    case SOL_ERR_INVALID_ARG: return "invalid argument (null pointer, size, NaN beta, workspace or alignment)";
    case SOL_ERR_UNSUPPORTED: return "unsupported configuration (head dim must be 128, block 64 or 128, mode 0 or 1)";
    case SOL_ERR_HIP: return "HIP runtime reported a launch error";
    case SOL_ERR_SCRATCH:
      return "the call needs more scratch than the allocation-free entry point holds (128 MiB)";
    default: return "unknown error code";
  }
}

int sol_attn_pool(const uint16_t* k, const uint16_t* v, float* kbar, float* vbar, int N, int H,
                  int d, int B, void* stream) {
  if (!k || !v || !kbar || !vbar) return SOL_ERR_INVALID_ARG;
  if (int r = check_shape(N, H, d)) return r;
  if (int r = check_block(B)) return r;
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(kbar, 16) || !aligned(vbar, 16))
    return SOL_ERR_INVALID_ARG;
  PoolArgs a{k, v, kbar, vbar, nullptr, nullptr, nullptr, N, H, B, cdiv(N, B), 0};
  return hip_status(launch_pool(a, (hipStream_t)stream));
}

int sol_attn_row_stats(const uint16_t* q, const float* kbar, float* mu, float* sigma, int N,
                       int Nk, int H, int d, int B, void* stream) {
  if (!q || !kbar || !mu || !sigma) return SOL_ERR_INVALID_ARG;
  if (Nk == 0) Nk = N;
  if (Nk < 0) return SOL_ERR_INVALID_ARG;
  if (int r = check_shape(N, H, d)) return r;
  if (int r = check_block(B)) return r;
  if (!aligned(q, 16) || !aligned(kbar, 16)) return SOL_ERR_INVALID_ARG;
  StatsArgs a{q, kbar, mu, sigma, N, H, cdiv(Nk, B)};
  return hip_status(launch_stats(a, (hipStream_t)stream));
}

int sol_attn_row_stats_moment(const uint16_t* q, const float* kbar, float* mu, float* sigma,
                              int N, int Nk, int H, int d, int B, void* workspace,
                              size_t ws_bytes, void* stream) {
  if (!q || !kbar || !mu || !sigma || !workspace) return SOL_ERR_INVALID_ARG;
  if (Nk == 0) Nk = N;
  if (Nk < 0) return SOL_ERR_INVALID_ARG;
  if (int r = check_shape(N, H, d)) return r;
  if (int r = check_block(B)) return r;
  if (!aligned(q, 16) || !aligned(kbar, 16) || !aligned(workspace, 256)) return SOL_ERR_INVALID_ARG;
  if (ws_bytes < (size_t)H * kMomentBytesPerHead) return SOL_ERR_INVALID_ARG;
  char* ws = (char*)workspace;
  const size_t c_bytes = (size_t)H * 128 * 128 * sizeof(uint16_t);
  MomentArgs ma{kbar, (uint16_t*)ws, (uint16_t*)(ws + c_bytes), (float*)(ws + 2 * c_bytes),
                (float*)(ws + 2 * c_bytes + (size_t)H * 128 * sizeof(float)), H, cdiv(Nk, B)};
  if (int r = hip_status(launch_moments(ma, (hipStream_t)stream))) return r;
  StatsMomentArgs sm{q, ma.chi, ma.clo, ma.mbar, mu, sigma, N, H};
  return hip_status(launch_stats_moment(sm, (hipStream_t)stream));
}

int fp8_quantize_rows(const uint16_t* x, uint8_t* q, float* scale, int64_t M, int K,
                      void* stream) {
  if (!x || !q || !scale || M <= 0 || K <= 0) return SOL_ERR_INVALID_ARG;
  if (K % 8 != 0) return SOL_ERR_UNSUPPORTED;
  if (!aligned(x, 16) || !aligned(q, 8)) return SOL_ERR_INVALID_ARG;
  Fp8QuantArgs a{x, q, scale, M, K};
  return hip_status(launch_quantize_rows(a, (hipStream_t)stream));
}

int fp8_gemm_rowscale(const uint8_t* a, const float* sa, const uint8_t* w, const float* sw,
                      uint16_t* y, int M, int N, int K, void* stream) {
  if (!a || !sa || !w || !sw || !y || M <= 0 || N <= 0 || K <= 0) return SOL_ERR_INVALID_ARG;
  if (K % 128 != 0 || N % 128 != 0) return SOL_ERR_UNSUPPORTED;
  if (!aligned(a, 16) || !aligned(w, 16) || !aligned(sw, 16) || !aligned(y, 16))
    return SOL_ERR_INVALID_ARG;
  Fp8GemmArgs g{};
  g.a = a; g.sa = sa; g.w = w; g.sw = sw; g.y = y; g.M = M; g.N = N; g.K = K;
  return hip_status(launch_fp8_gemm(g, (hipStream_t)stream));
}

int na3d_forward(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* out,
                 float* lse, int T, int Y, int X, int H, int d, int kt, int ky, int kx,
                 void* stream) {
  if (!q || !k || !v || !out) return SOL_ERR_INVALID_ARG;
  if (T <= 0 || Y <= 0 || X <= 0 || H <= 0) return SOL_ERR_INVALID_ARG;
  if (d != 128) return SOL_ERR_UNSUPPORTED;
  auto odd_fits = [](int w, int len) { return w >= 1 && (w & 1) && w <= len; };
  if (!odd_fits(kt, T) || !odd_fits(ky, Y) || !odd_fits(kx, X)) return SOL_ERR_INVALID_ARG;
  if (kx > 25) return SOL_ERR_UNSUPPORTED;
  if ((long long)T * Y * X > (1LL << 31) / 128) return SOL_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
    return SOL_ERR_INVALID_ARG;
  Na3dArgs a{q, k, v, out, lse, T, Y, X, H, kt, ky, kx};
  return hip_status(launch_na3d(a, (hipStream_t)stream));
}

size_t sol_attn_workspace_size(int N, int Nk, int H, int d, int B, int mode) {
  if (Nk == 0) Nk = N;
  if (N <= 0 || Nk <= 0 || H <= 0 || d != 128) return 0;
  if (mode != SOL_DENSE && mode != SOL_SPARSE) return 0;
  if (mode == SOL_SPARSE && check_block(B)) return 0;
  return make_plan(N, Nk, H, B, mode).bytes;
}

int sol_attn_forward(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* out,
                     float* lse, int N, int H, int d, int B, float beta, int mode, int Nk,
                     void* workspace, size_t ws_bytes, void* stream) {
  if (Nk == 0) Nk = N;
  if (int r = check_forward(q, k, v, out, N, H, d, B, beta, mode, Nk)) return r;
  const Plan p = make_plan(N, Nk, H, B, mode);
  if (p.bytes > 0 && (!workspace || ws_bytes < p.bytes || !aligned(workspace, 256)))
    return SOL_ERR_INVALID_ARG;
  return forward_launch(q, k, v, out, lse, N, H, B, beta, mode, Nk, p, workspace, stream);
}

int sol_attn_forward_noalloc(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                             uint16_t* out, float* lse, int N, int H, int d, int B, float beta,
                             int mode, int Nk, void* stream) {
  if (Nk == 0) Nk = N;
  if (int r = check_forward(q, k, v, out, N, H, d, B, beta, mode, Nk)) return r;
  const Plan p = make_plan(N, Nk, H, B, mode);
  if (p.bytes > kScratchBytes) return SOL_ERR_SCRATCH;
  void* ws = nullptr;
  if (p.bytes > 0) {
    if (int r = scratch_of_stream_device(stream, &ws)) return r;
  }
  return forward_launch(q, k, v, out, lse, N, H, B, beta, mode, Nk, p, ws, stream);
}

int sol_attn_tile_schedule(const uint16_t* q, const uint16_t* k, const uint16_t* v, int* work,
                           int* order, int N, int H, int d, int B, float beta, int Nk,
                           void* workspace, size_t ws_bytes, void* stream) {
  if (Nk == 0) Nk = N;
  if (!work || !order || !aligned(work, 4) || !aligned(order, 4)) return SOL_ERR_INVALID_ARG;
  if (isinf(beta) && beta < 0) return SOL_ERR_INVALID_ARG;  // dense: no selection to count
  // the forward's checks; there is no output here, so q stands in for it
  if (int r = check_forward(q, k, v, q, N, H, d, B, beta, SOL_SPARSE, Nk)) return r;
  if (cdiv(N, 128) > kOrderMaxTiles) return SOL_ERR_UNSUPPORTED;
  const Plan p = make_plan(N, Nk, H, B, SOL_SPARSE);
  if (!workspace || ws_bytes < p.bytes || !aligned(workspace, 256)) return SOL_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  Routing rt;
  if (int r = route(q, k, v, N, H, B, Nk, p, (char*)workspace, s, &rt)) return r;
  TileOrderArgs ta{q, rt.pool.khi, rt.pool.klo, rt.mu, rt.sigma, work, order, beta, N, H,
                   p.sp.nb, p.sp.nb_pad, cdiv(N, 128)};
  return hip_status(launch_tile_order(ta, s));
}

size_t sol_attn_shard_workspace_size(int N, int Nk, int nb_all, int H, int d, int B,
                                     float beta) {
  if (N <= 0 || Nk <= 0 || H <= 0 || d != 128 || check_block(B) || isnan(beta)) return 0;
  const bool sparse = !(isinf(beta) && beta < 0);
  if (sparse && nb_all < cdiv(Nk, B)) return 0;
  return make_shard_plan(N, Nk, nb_all, H, B, sparse).bytes;
}

int sol_attn_forward_shard(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                           const float* kbar_all, float* part_o, float* part_ml, int N,
                           int Nk, int nb_all, int H, int d, int B, float beta,
                           void* workspace, size_t ws_bytes, void* stream) {
  if (!q || !k || !v || !part_o || !part_ml) return SOL_ERR_INVALID_ARG;
  if (int r = check_shape(N, H, d)) return r;
  if (Nk <= 0) return SOL_ERR_INVALID_ARG;
  if (int r = check_block(B)) return r;
  if (isnan(beta)) return SOL_ERR_INVALID_ARG;
  const bool sparse = !(isinf(beta) && beta < 0);
  if (sparse && (!kbar_all || nb_all < cdiv(Nk, B) || !aligned(kbar_all, 16)))
    return SOL_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(part_o, 16) ||
      !aligned(part_ml, 8))
    return SOL_ERR_INVALID_ARG;
  const ShardPlan p = make_shard_plan(N, Nk, nb_all, H, B, sparse);
  if (p.bytes > 0 && (!workspace || ws_bytes < p.bytes || !aligned(workspace, 256)))
    return SOL_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;

  FwdArgs f{};
  f.q = q; f.k = k; f.v = v; f.out = nullptr; f.lse = nullptr;
  f.beta = beta; f.N = N; f.Nk = Nk; f.H = H;
  f.nb = p.nb; f.nb_pad = p.nb_pad;
  f.n_qt = cdiv(N, 128);
  f.splits = 1; f.tiles_per_split = p.nb;
  f.total = H * f.n_qt;
  f.part_o = part_o; f.part_ml = part_ml;
  if (sparse) {
    // local blocks pooled for routing and the Taylor term; thresholds from
    // the pooled keys of the whole sequence
    PoolArgs pa{k, v, (float*)(ws + p.off_kbar), (float*)(ws + p.off_vbar),
                (uint16_t*)(ws + p.off_vsum), (uint16_t*)(ws + p.off_khi),
                (uint16_t*)(ws + p.off_klo), Nk, H, B, p.nb, p.nb_pad};
    if (int r = hip_status(launch_pool(pa, s))) return r;
    float* mu = (float*)(ws + p.off_mu);
    float* sigma = (float*)(ws + p.off_sigma);
    if (p.moments) {
      MomentArgs ma{kbar_all, (uint16_t*)(ws + p.off_chi), (uint16_t*)(ws + p.off_clo),
                    (float*)(ws + p.off_mbar), (float*)(ws + p.off_mpart), H, nb_all};
      if (int r = hip_status(launch_moments(ma, s))) return r;
      StatsMomentArgs sm{q, ma.chi, ma.clo, ma.mbar, mu, sigma, N, H};
      if (int r = hip_status(launch_stats_moment(sm, s))) return r;
    } else {
      StatsArgs sa{q, kbar_all, mu, sigma, N, H, nb_all};
      if (int r = hip_status(launch_stats(sa, s))) return r;
    }
    f.khi = pa.khi; f.klo = pa.klo; f.vsumT = pa.vsumT; f.mu = mu; f.sigma = sigma;
    if (p.order) {
      TileOrderArgs ta{q, pa.khi, pa.klo, mu, sigma, (int*)(ws + p.off_work),
                       (int*)(ws + p.off_order), beta, N, H, p.nb, p.nb_pad, f.n_qt};
      if (int r = hip_status(launch_tile_order(ta, s))) return r;
      f.order = ta.order;
    }
  }
  return hip_status(sparse ? launch_forward(f, B, s) : launch_forward_dense(f, s));
}

int sol_attn_combine_partials(const float* part_o, const float* part_ml, int S, uint16_t* out,
                              float* lse, int N, int H, int d, void* stream) {
  if (!part_o || !part_ml || !out || S <= 0) return SOL_ERR_INVALID_ARG;
  if (int r = check_shape(N, H, d)) return r;
  if (!aligned(part_o, 16) || !aligned(part_ml, 8) || !aligned(out, 16)) return SOL_ERR_INVALID_ARG;
  CombineArgs c{part_o, part_ml, out, lse, N, H, S};
  return hip_status(launch_combine(c, (hipStream_t)stream));
}

int attn_lse_merge(const uint16_t* out_a, const float* lse_a, const uint16_t* out_b,
                   const float* lse_b, uint16_t* out, float* lse, int N, int H, int d,
                   void* stream) {
  if (!out_a || !lse_a || !out_b || !lse_b || !out || !lse) return SOL_ERR_INVALID_ARG;
  if (int r = check_shape(N, H, d)) return r;
  if (!aligned(out_a, 16) || !aligned(out_b, 16) || !aligned(out, 16)) return SOL_ERR_INVALID_ARG;
  MergeArgs a{out_a, lse_a, out_b, lse_b, out, lse, N, H};
  return hip_status(launch_merge(a, (hipStream_t)stream));
}

int sol_attn_proxy_scores(const uint16_t* q, const float* kbar, float* p, int row0, int nrows,
                          int N, int Nk, int H, int d, int B, void* stream) {
  if (!q || !kbar || !p) return SOL_ERR_INVALID_ARG;
  if (Nk == 0) Nk = N;
  if (Nk < 0 || row0 < 0 || nrows <= 0 || row0 + nrows > N) return SOL_ERR_INVALID_ARG;
  if (int r = check_shape(N, H, d)) return r;
  if (int r = check_block(B)) return r;
  if (!aligned(q, 16) || !aligned(kbar, 16)) return SOL_ERR_INVALID_ARG;
  ProxyArgs a{q, kbar, p, row0, nrows, N, H, cdiv(Nk, B)};
  return hip_status(launch_proxy(a, (hipStream_t)stream));
}

int sol_attn_block_mask(const uint16_t* q, const float* kbar, const float* mu, const float* sigma,
                        float beta, int row0, int nrows, int N, int Nk, int H, int d, int B,
                        uint8_t* mask, int64_t* counts, void* stream) {
  if (!q || !kbar || !mu || !sigma || !counts) return SOL_ERR_INVALID_ARG;
  if (Nk == 0) Nk = N;
  if (Nk < 0 || row0 < 0 || nrows <= 0 || row0 + nrows > N || (row0 % 128) != 0)
    return SOL_ERR_INVALID_ARG;
  if (isnan(beta)) return SOL_ERR_INVALID_ARG;
  if (int r = check_shape(N, H, d)) return r;
  if (int r = check_block(B)) return r;
  if (!aligned(q, 16) || !aligned(kbar, 16) || !aligned(counts, 8)) return SOL_ERR_INVALID_ARG;
  MaskArgs a{q, kbar, mu, sigma, beta, mask, (unsigned long long*)counts, row0, nrows, N, H,
             cdiv(Nk, B)};
  return hip_status(launch_mask(a, (hipStream_t)stream));
}

}  // extern "C"

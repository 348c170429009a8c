// gemm.hip -- launcher of the bf16 MFMA GEMM (the tile itself is in
// gemm_tile.h): one work-group per tile and K slice; the output tiles leave
// with streaming stores (read by the next launch, not by this one).
#include "gemm_tile.h"

namespace df2 {
using namespace gemm;
namespace {

template <int BM, int BN, int S, int NW, int ISSUE>
__global__ __launch_bounds__(NW * 64) void gemm_dma_kernel(Problem Pb) {
  run_tile<BM, BN, S, NW, ISSUE, true>(Pb, blockIdx.x, gridDim.x);
}

// One dense problem, its fields passed as separate arguments: an aggregate
// passed by value is not preloaded into SGPRs, scalars and pointers are
// (all 48 bytes of these arrive preloaded).
template <int BM, int BN, int S, int NW, int ISSUE>
__global__ __launch_bounds__(NW * 64) void gemm_dense_kernel(const uint16_t* x, const uint16_t* w, float* out,
                                                             int M, int N, int K, int ksplit, int ldx, int ldo) {
  DenseProblem D;
  D.x = x;
  D.w = w;
  D.out = out;
  D.M = M;
  D.N = N;
  D.K = K;
  D.ksplit = ksplit;
  D.ldx = ldx;
  D.ldo = ldo;
  run_tile_dense<BM, BN, S, NW, ISSUE, true>(D, blockIdx.x);
}

}  // namespace

// Raise the dynamic-LDS limit of a kernel once (idempotent; a race between
// threads only repeats the call).
hipError_t gemm::allow_lds(const void* fn, int bytes, bool& done) {
  if (done) return hipSuccess;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done = true;
  return e;
}

hipError_t gemm::make_problem(const GemmSeg* segs, int nseg, int K, int ksplit, int bm, int bn,
                              Problem& P, int& tiles) {
  tiles = 0;
  P.nseg = 0;
  if (nseg > kMaxSeg || K % BK != 0 || ksplit < 1 || ksplit > K / BK) return hipErrorInvalidValue;
  for (int i = 0; i < nseg; ++i) {
    if (segs[i].M <= 0) continue;
    GemmSeg s = segs[i];
    // lane offsets are 32-bit and must be able to point past the data for
    // the whole K walk; W tiles must not straddle w0 / w1
    const uint64_t lim = (1ull << 32) - 16u - 2u * (uint64_t)K;
    if ((uint64_t)s.x_rows * (uint64_t)s.ldx * 2u > lim) return hipErrorInvalidValue;
    if ((uint64_t)s.N * (uint64_t)K * 2u > lim) return hipErrorInvalidValue;
    if (s.n0 < s.N && s.n0 % bn != 0) return hipErrorInvalidValue;
    if (s.grp_rows < 0 || (s.grp_rows > 0 && s.grp_stride < s.grp_rows)) return hipErrorInvalidValue;
    s.tiles_m = (s.M + bm - 1) / bm;
    s.tiles_n = (s.N + bn - 1) / bn;
    P.s[P.nseg] = s;
    P.tile_begin[P.nseg] = tiles;
    tiles += s.tiles_m * s.tiles_n;
    P.nseg++;
  }
  for (int i = P.nseg; i <= kMaxSeg; ++i) P.tile_begin[i] = tiles;
  P.K = K;
  P.ksplit = ksplit;
  return hipSuccess;
}

hipError_t launch_gemm(const GemmSeg* segs, int nseg, int K, int ksplit, const GemmTiling& t,
                       const char* tag, hipStream_t stream) {
  Problem P;
  int tiles = 0;
  hipError_t pe = make_problem(segs, nseg, K, ksplit, t.bm, t.bn, P, tiles);
  if (pe != hipSuccess) return pe;
  if (tiles == 0) return hipSuccess;
  dim3 grid((unsigned)(tiles * ksplit));
  ProfileScope ps(tag, stream);
  // one dense problem whose sizes fit the compact arguments: the kernel
  // whose arguments are all preloaded
  const GemmSeg& s0 = P.s[0];
  const bool dense = P.nseg == 1 && !s0.gather && s0.grp_rows == 0 && s0.gate == 0 && s0.n0 >= s0.N &&
                     s0.x_rows == s0.M && s0.ldx <= INT32_MAX && s0.ldo <= INT32_MAX &&
                     (P.ksplit == 1 || s0.out_kstride == (int64_t)s0.M * s0.ldo);
  DenseProblem D{};
  if (dense) {
    D.x = s0.x;
    D.w = s0.w0;
    D.out = s0.out;
    D.M = s0.M;
    D.N = s0.N;
    D.K = P.K;
    D.ksplit = P.ksplit;
    D.ldx = (int)s0.ldx;
    D.ldo = (int)s0.ldo;
  }
#define DF2_GEMM_LAUNCH(BMV, BNV, SV, NWV, IV)                                                          \
  if (t.bm == BMV && t.bn == BNV && t.stages == SV && t.waves == NWV && t.issue == IV) {               \
    constexpr int kLds = SV * (BMV + BNV) * BK * 2;                                                    \
    if (dense) {                                                                                       \
      static bool done_d = false;                                                                      \
      hipError_t e = allow_lds((const void*)gemm_dense_kernel<BMV, BNV, SV, NWV, IV>, kLds, done_d);   \
      if (e != hipSuccess) return e;                                                                   \
      return launch(gemm_dense_kernel<BMV, BNV, SV, NWV, IV>, grid, dim3(NWV * 64), kLds, stream, ps, D.x, D.w, \
                    D.out, D.M, D.N, D.K, D.ksplit, D.ldx, D.ldo);                                              \
    }                                                                                                  \
    static bool done = false;                                                                          \
    hipError_t e = allow_lds((const void*)gemm_dma_kernel<BMV, BNV, SV, NWV, IV>, kLds, done);         \
    if (e != hipSuccess) return e;                                                                     \
    return launch(gemm_dma_kernel<BMV, BNV, SV, NWV, IV>, grid, dim3(NWV * 64), kLds, stream, ps, P);  \
  }
  DF2_GEMM_LAUNCH(64, 128, 3, 4, 1)    // H, projection at small batches
  DF2_GEMM_LAUNCH(64, 128, 4, 8, 3)    // the conv's taps below 1,024 rows
  DF2_GEMM_LAUNCH(128, 128, 4, 8, 3)   // projection, per-token tables, the conv's taps from 1,024 rows
  DF2_GEMM_LAUNCH(256, 128, 3, 8, 3)   // projection with more than one round of 128 x 128 tiles
#undef DF2_GEMM_LAUNCH
  return hipErrorInvalidValue;
}

}  // namespace df2

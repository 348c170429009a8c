// gemm.hip -- out = gate(X W^T) with bf16 operands on the gfx950 matrix
// cores (v_mfma_f32_16x16x32_bf16), fp32 accumulation.
//
// Used for the rank-r projections of the path selector (A(tok) = W_A E[tok],
// B(tok) = W_B E[tok], H = gate(W_H h_t); "DFlash 2: Keep Drafting Parallel",
// section "A lightweight path selector") and for the tap corrections of the
// two-tap conv (c_t = W x_t; section "A lightweight local convolution").
// Both operands are K-contiguous rows (X: [M, K], W: [N, K]), so every lane
// feeds the MFMA with 16 contiguous bytes of one row.
//
// Tiling: work-group = 4 waves (2 x 2), tile BM x 128 x 64 (BM = 128 or 64),
// double-buffered LDS with rows padded to 144 bytes (conflict-free 16-byte
// fragment reads), and a ring of P register-staged K-tiles so that P tiles
// are in flight while the MFMAs of the current one run (one tile of MFMA
// work is far shorter than a memory round trip).  X rows may be gathered through an index list (candidate tokens
// into the embedding table).  Up to three independent problems share one
// launch.  An optional K split writes per-slice partial products (no
// atomics; the consumer sums the slices in a fixed order).
// Work-groups are renumbered so that each XCD runs a contiguous range of
// tiles: the N-tiles of one M-block then share that XCD's L2 for X.
#include "df2_device.h"
#include "df2_internal.h"

namespace df2 {
namespace {

constexpr int BN = 128, BK = 64, LDSW = BK + 8;  // LDS row = 72 bf16 = 144 bytes
constexpr int kThreads = 256;
constexpr int kXcds = 8;

struct Problem {
  GemmSeg s[3];
  int tile_begin[4];
  int nseg;
  int K;       // full reduction length; W rows are K apart
  int ksplit;
  int kslice;  // K elements per slice (multiple of BK)
};

__device__ __forceinline__ float apply_gate(float z, int gate) {
  return gate == 1 ? 1.0f / (1.0f + expf(-z)) : z;
}

template <int BM, int P>
__global__ __launch_bounds__(kThreads) void gemm_kernel(Problem Pb) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr int XCH = BM * BK / 8 / kThreads;
  constexpr int WCH = BN * BK / 8 / kThreads;
  __shared__ __attribute__((aligned(16))) uint16_t sX[2][BM * LDSW];
  __shared__ __attribute__((aligned(16))) uint16_t sW[2][BN * LDSW];

  // XCD-aware numbering (work-group i runs on XCD i % 8).  Without a K
  // split, each XCD takes a contiguous range of tiles, so the N-tiles of one
  // M-block share that XCD's L2 for their X rows.  With a K split, the slice
  // index is the fastest-varying part of the id, so each XCD holds one
  // K-slice of X and W in its L2 and every byte comes from HBM once.
  const int nb = gridDim.x;
  int bid = blockIdx.x;
  int tile, ks;
  if (Pb.ksplit == 1) {
    const int full = nb / kXcds * kXcds;
    if (bid < full) bid = (bid % kXcds) * (full / kXcds) + bid / kXcds;
    tile = bid;
    ks = 0;
  } else {
    tile = bid / Pb.ksplit;
    ks = bid % Pb.ksplit;
  }
  int si = 0;
  while (si + 1 < Pb.nseg && tile >= Pb.tile_begin[si + 1]) ++si;
  const GemmSeg& S = Pb.s[si];
  const int local = tile - Pb.tile_begin[si];
  const int m0 = (local / S.tiles_n) * BM, n0 = (local % S.tiles_n) * BN;
  const int k_begin = ks * Pb.kslice;
  const int nk = Pb.kslice / BK;

  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int wm = wave >> 1, wn = wave & 1;

  // Per-thread source rows for the 16-byte chunks it stages.  Loads are
  // unconditional (so the compiler can count them and keep several K-tiles
  // in flight): rows outside the problem read row 0 and are replaced by
  // zeros when staged into LDS.
  const uint16_t* xp[XCH];
  const uint16_t* wp[WCH];
  bool xv[XCH], wv[WCH];
#pragma unroll
  for (int i = 0; i < XCH; ++i) {
    int c = tid + i * kThreads, row = c / (BK / 8), col = (c % (BK / 8)) * 8;
    int m = m0 + row;
    int64_t src = 0;
    bool ok = false;
    if (m < S.M) {
      src = S.gather ? (int64_t)S.gather[m] : (int64_t)m;
      ok = src >= 0 && src < S.x_rows;
      if (!ok) src = 0;
    }
    xv[i] = ok;
    xp[i] = S.x + src * S.ldx + k_begin + col;
  }
#pragma unroll
  for (int i = 0; i < WCH; ++i) {
    int c = tid + i * kThreads, row = c / (BK / 8), col = (c % (BK / 8)) * 8;
    int n = n0 + row;
    wv[i] = n < S.N;
    const uint16_t* p = !wv[i] ? S.w0 : n < S.n0 ? S.w0 + (int64_t)n * Pb.K
                                               : S.w1 + (int64_t)(n - S.n0) * Pb.K;
    wp[i] = p + k_begin + col;
  }

  // Register ring of P staged K-tiles: tile t lives in slot t % P.  While
  // the MFMAs of tile k run from LDS, tiles k+1 .. k+P are in flight.
  // Tiles past the end re-read the last tile (never stored).
  u32x4 rx[P][XCH], rw[P][WCH];
  auto gload = [&](int kt, u32x4 (&dx)[XCH], u32x4 (&dw)[WCH]) {
    const int off = (kt < nk ? kt : nk - 1) * BK;
#pragma unroll
    for (int i = 0; i < XCH; ++i) dx[i] = *(const u32x4*)(xp[i] + off);
#pragma unroll
    for (int i = 0; i < WCH; ++i) dw[i] = *(const u32x4*)(wp[i] + off);
  };
  const u32x4 z4 = u32x4{0u, 0u, 0u, 0u};
  auto sstore = [&](int buf, const u32x4 (&dx)[XCH], const u32x4 (&dw)[WCH]) {
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      int c = tid + i * kThreads, row = c / (BK / 8), col = (c % (BK / 8)) * 8;
      *(u32x4*)&sX[buf][row * LDSW + col] = xv[i] ? dx[i] : z4;
    }
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
      int c = tid + i * kThreads, row = c / (BK / 8), col = (c % (BK / 8)) * 8;
      *(u32x4*)&sW[buf][row * LDSW + col] = wv[i] ? dw[i] : z4;
    }
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int t = 0; t < P; ++t) gload(t, rx[t], rw[t]);
  sstore(0, rx[0], rw[0]);
  gload(P, rx[0], rw[0]);
  __syncthreads();
  const int fr = lane & 15, fk = (lane >> 4) * 8;
  // nk is a multiple of P: the unrolled group below has no guards, so the
  // compiler can count outstanding loads and wait only for the tile it
  // stores.  The last step stores a tile nobody reads.
  for (int k0 = 0; k0 < nk; k0 += P) {
#pragma unroll
    for (int st = 0; st < P; ++st) {
      const int kt = k0 + st;
      const int buf = kt & 1;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        bf16x8 a[FM], b[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
          a[i] = *(const bf16x8*)&sX[buf][(wm * WM + i * 16 + fr) * LDSW + s * 32 + fk];
#pragma unroll
        for (int j = 0; j < FN; ++j)
          b[j] = *(const bf16x8*)&sW[buf][(wn * WN + j * 16 + fr) * LDSW + s * 32 + fk];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
      }
      const int nx = (st + 1) % P;   // slot of tile kt + 1 (a constant once unrolled)
      sstore(buf ^ 1, rx[nx], rw[nx]);
      gload(kt + 1 + P, rx[nx], rw[nx]);
      __syncthreads();
    }
  }

  // D[i][j] of a 16x16 tile: lane holds column (lane & 15), rows 4*(lane>>4)+e
  float* out = S.out + (int64_t)ks * S.out_kstride;
  const int gate = S.gate;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = n0 + wn * WN + j * 16 + fr;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + wm * WM + i * 16 + (lane >> 4) * 4 + e;
        if (m < S.M && n < S.N) out[(int64_t)m * S.ldo + n] = apply_gate(acc[i][j][e], gate);
      }
    }
}

}  // namespace

hipError_t launch_gemm(const GemmSeg* segs, int nseg, int K, int ksplit, int bm,
                       const char* tag, hipStream_t stream) {
  Problem P;
  int tiles = 0;
  P.nseg = 0;
  for (int i = 0; i < nseg; ++i) {
    if (segs[i].M <= 0) continue;
    GemmSeg s = segs[i];
    s.tiles_m = (s.M + bm - 1) / bm;
    s.tiles_n = (s.N + BN - 1) / BN;
    P.s[P.nseg] = s;
    P.tile_begin[P.nseg] = tiles;
    tiles += s.tiles_m * s.tiles_n;
    P.nseg++;
  }
  P.tile_begin[P.nseg] = tiles;
  if (tiles == 0) return hipSuccess;
  P.K = K;
  P.ksplit = ksplit;
  P.kslice = K / ksplit;
  dim3 grid((unsigned)(tiles * ksplit)), block(kThreads);
  ProfileScope ps(tag, stream);
  // pipeline depth: the largest of 4, 5, 2, 1 that divides the K-tile count
  const int nk = P.kslice / BK;
  const int depth = nk % 4 == 0 ? 4 : nk % 5 == 0 ? 5 : nk % 2 == 0 ? 2 : 1;
#define DF2_GEMM_LAUNCH(BMV, PV) gemm_kernel<BMV, PV><<<grid, block, 0, stream>>>(P)
  if (bm == 128) {
    if (depth == 4) DF2_GEMM_LAUNCH(128, 4);
    else if (depth == 5) DF2_GEMM_LAUNCH(128, 5);
    else if (depth == 2) DF2_GEMM_LAUNCH(128, 2);
    else DF2_GEMM_LAUNCH(128, 1);
  } else {
    if (depth == 4) DF2_GEMM_LAUNCH(64, 4);
    else if (depth == 5) DF2_GEMM_LAUNCH(64, 5);
    else if (depth == 2) DF2_GEMM_LAUNCH(64, 2);
    else DF2_GEMM_LAUNCH(64, 1);
  }
#undef DF2_GEMM_LAUNCH
  return hipGetLastError();
}

}  // namespace df2

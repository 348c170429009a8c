// gemm_tile.h -- bf16 MFMA GEMM tile (out = gate(X W^T), fp32 accumulation).
// The tile body is a device function so that a persistent kernel can run
// GEMM tiles among other work; gemm.hip holds the stand-alone launcher.
//
// Used for the rank-r projections of the path selector (A(tok) = W_A E[tok],
// B(tok) = W_B E[tok], H = gate(W_H h_t); "DFlash 2: Keep Drafting Parallel",
// section "A lightweight path selector") and for the tap corrections of the
// two-tap conv (c_t = W x_t; section "A lightweight local convolution").
// Both operands are K-contiguous rows (X: [M, K], W: [N, K]), so every lane
// feeds the MFMA with 16 contiguous bytes of one row.
//
// Tiling: work-group = 4 or 8 waves (2 x 2 or 2 x 4), tile BM x BN (BM = 64
// or 128; BN = 128 in the instantiations), K-tiles of 64.  X rows may be
// gathered through an index list (candidate tokens into the embedding table).  Up to four independent
// problems share one launch.  An optional K split writes per-slice partial
// products (no atomics; the consumer sums the slices in a fixed order).
// Work-groups are renumbered so that each XCD runs a contiguous range of
// tiles (the N-tiles of one M-block then share that XCD's L2 for X), or,
// with a K split, so that the slice index varies fastest.
// Files that run these tiles are compiled with the VGPR form of the MFMA
// instructions (gemm.hip, cycle_fused.hip): the
// accumulators live in ordinary VGPRs, which keeps the accumulate chain free
// of register copies.
#pragma once

#include "df2_device.h"
#include "df2_internal.h"
#include "mfma_tile.h"

namespace df2 {

// dynamic LDS of the GEMM (declared outside any anonymous namespace: an
// extern with internal linkage keeps the host-side launch stub from being
// emitted)
extern __shared__ __attribute__((aligned(16))) uint8_t dyn_lds[];

namespace gemm {

using mfma::BK;
constexpr int kXcds = 8;

constexpr int kMaxSeg = 4;

// The scalars every work-group needs first lead the kernel arguments, so
// that one scalar load fetches them all (the segment's fields follow in a
// second round trip, once the segment index is known).
struct Problem {
  int ksplit;  // slice s covers K-tiles [s nkt / ksplit, (s + 1) nkt / ksplit)
  int K;       // full reduction length; W rows are K apart
  int nseg;
  int tile_begin[kMaxSeg + 1];   // entries from nseg on hold the tile total
  GemmSeg s[kMaxSeg];
};

__device__ __forceinline__ float apply_gate(float z, int gate) {
  return gate == 1 ? 1.0f / (1.0f + expf(-z)) : z;
}

// The K-tiles are copied by direct buffer-to-LDS loads (no register
// staging) into S LDS stages, S - 1 of them in flight while the MFMAs of the
// current one run; one barrier per K-tile (where the next copies are issued
// within a K step: ISSUE below).  The stage layout, the chunk
// swizzle and the load helper are in mfma_tile.h.
using mfma::load_lds16;
using mfma::swz;
using mfma::vmcnt_imm;

// The tile of work-group `bid` of a grid of `nb` (the body of the GEMM
// kernel; NW waves per work-group: 2 x 2 (NW = 4) or 2 x 4 (NW = 8)).
// ISSUE 3: the ping-pong loop of mfma_tile.h (NW = 8, waves in two
// alternating groups).  ISSUE 0-2: where in a K step the copies of tile t + S - 1 are issued (into
// the stage read in step t - 1, which every wave left before this step's
// barrier): 0 right after the barrier (the longest lead: best for the
// conv's few-K-tile, feed-bound tiles), 1 between the two halves of the
// tile's MFMAs, 2 after them (the copy queue is often full, and an issue
// that stalls then overlaps the matrix pipe's work instead of delaying it:
// per K-tile of the batch-32 projection, issuing first spent 244 of 1,237
// cycles in the issue; 55.7 -> 47.5 us alone).  Measured on one box, the
// batch-32 / block-16 step was 0.5220 ms with 0 everywhere, 0.5239 with 2
// and 0.5206 with 1 (the cycle without the conv 132.5 / 128.6 / 129.0 us).
// The tile itself: product rows m0 .. m0 + BM - 1 and columns n0 .. n0 + BN
// - 1 of one segment, K slice ks of ksplit (every argument a scalar).
// STREAM: the output tile leaves with nontemporal stores, which do not keep
// the written lines in the caches.  A stand-alone launch's outputs are read
// by a later kernel, so nothing is lost, and each of its lines that stays
// dirty in an XCD's L2 is written back when the kernel ends, after the last
// work-group.  Measured on the batch-32 / block-16 step (together with the
// conv epilogue's streamed y): 0.4862-0.4867 -> 0.4638-0.4645 ms; the stress
// cycle 861 -> 828 us.  The persistent cycle, whose consumers read the tiles
// in the same launch, keeps cached stores (streamed: 90.0 -> 92.7 us per
// batch-1 / block-16 cycle).
template <int BM, int BN, int S, int NW, int ISSUE, bool STREAM>
__device__ __forceinline__ void tile_core(const uint16_t* sx, const int32_t* sgather, int x_rows, int ldx, int M,
                                          int N, int sn0, const uint16_t* w0, const uint16_t* w1, float* sout,
                                          int64_t ldo, int64_t out_kstride, int gate, int grows, int gstride, int K,
                                          int m0, int n0, int ks, int ksplit) {
  static_assert(BM % (8 * NW) == 0 && BN % (8 * NW) == 0, "whole load instructions per wave");
  static_assert(ISSUE != 3 || NW == 8, "two alternating groups of four waves");
  static_assert((BM / 2) % 16 == 0 && (BN / (NW / 2)) % 16 == 0, "whole 16 x 16 blocks per wave");
  constexpr int kThreads = NW * 64;
  constexpr int WCOL = NW / 2;                  // waves along N
  constexpr int WM = BM / 2, WN = BN / WCOL;
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr int ALD = BM / (8 * NW), BLD = BN / (8 * NW);   // load instructions per wave per stage
  constexpr int LPW = ALD + BLD;
  constexpr int STAGE = (BM + BN) * BK * 2;     // bytes
  // product row -> row of the gather list / x and of out
  auto phys = [&](int m) { return grows > 0 ? (m / grows) * gstride + m % grows : m; };
  const int nkt = K / BK;
  const int kt0 = ks * nkt / ksplit, kt1 = (ks + 1) * nkt / ksplit;
  const int k_begin = kt0 * BK;
  const int nk = kt1 - kt0;
  const int wave = wave_id(), lane = lane_id();
  const int wm = wave / WCOL, wn = wave % WCOL;

  const bool from_w0 = n0 < sn0;
  const uint16_t* wbase = from_w0 ? w0 + (int64_t)n0 * K : w1 + (int64_t)(n0 - sn0) * K;
  const int wrows = (from_w0 ? (sn0 < N ? sn0 : N) : N) - n0;
  // in 64 bits: rows x ldx x 2 exceeds INT_MAX for tables over 2 GiB (the
  // launcher keeps it under 2^32 - 2K - 16)
  const uint32_t xbytes = (uint32_t)((uint64_t)(uint32_t)x_rows * (uint64_t)(uint32_t)ldx * 2u);
  const uint32_t wbytes = (uint32_t)((int64_t)wrows * K * 2);
  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc((void*)sx, 0, (int)xbytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc((void*)wbase, 0, (int)wbytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t xnone = __builtin_amdgcn_make_buffer_rsrc((void*)sx, 0, 0, kBufferWord3);
  const __amdgpu_buffer_rsrc_t wnone = __builtin_amdgcn_make_buffer_rsrc((void*)wbase, 0, 0, kBufferWord3);
  // out of range for the whole K walk, whether or not the range check adds
  // the scalar offset (the launcher keeps bytes + 2K + 16 <= 2^32)
  const uint32_t kOut = 0xFFFFFFF0u - (uint32_t)K * 2u;

  // lane offsets of this wave's load instructions: instruction a fills rows
  // 8 (wave + NW a) .. + 7 of the X tile, b likewise of the W tile.  X rows
  // come through the gather list when there is one: its entries are loaded
  // unconditionally (clamped row) so that all of them are in flight at once.
  const int sub = lane >> 3, slot = lane & 7;
  uint32_t xo[ALD], wo[BLD];
  int src[ALD];
#pragma unroll
  for (int a = 0; a < ALD; ++a) {
    const int m = m0 + 8 * (wave + NW * a) + sub;
    src[a] = phys(m < M ? m : M - 1);
  }
  if (sgather) {
#pragma unroll
    for (int a = 0; a < ALD; ++a) src[a] = sgather[src[a]];
  }
#pragma unroll
  for (int a = 0; a < ALD; ++a) {
    const int row = 8 * (wave + NW * a) + sub;
    const int c = slot ^ swz(row);
    const bool ok = m0 + row < M && src[a] >= 0 && src[a] < x_rows;
    xo[a] = ok ? (uint32_t)(((int64_t)src[a] * ldx + k_begin + c * 8) * 2) : kOut;
  }
#pragma unroll
  for (int b = 0; b < BLD; ++b) {
    const int row = 8 * (wave + NW * b) + sub;
    const int c = slot ^ swz(row);
    wo[b] = row < wrows ? (uint32_t)(((int64_t)row * K + k_begin + c * 8) * 2) : kOut;
  }
  // K-tile t goes to stage t % S; tiles past the end read nothing (empty
  // resources: zeros, no traffic) so that every step issues the same loads
  auto issue = [&](int t) {
    const bool in = t < nk;
    uint8_t* sb = dyn_lds + (t % S) * STAGE;
    const int so = __builtin_amdgcn_readfirstlane(in ? t * BK * 2 : 0);
    const __amdgpu_buffer_rsrc_t rx = in ? xres : xnone, rw = in ? wres : wnone;
#pragma unroll
    for (int a = 0; a < ALD; ++a)
      load_lds16(rx, sb + (wave + NW * a) * 8 * 128, xo[a], so);
#pragma unroll
    for (int b = 0; b < BLD; ++b)
      load_lds16(rw, sb + BM * 128 + (wave + NW * b) * 8 * 128, wo[b], so);
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int fr = lane & 15, fq = lane >> 4;
  // fragment byte offsets inside a stage (rows fixed per lane, chunk 4 s + fq)
  int ao[FM][2], bo[FN][2];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int r = wm * WM + i * 16 + fr;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) ao[i][s2] = r * 128 + 16 * ((4 * s2 + fq) ^ swz(r));
  }
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int r = wn * WN + j * 16 + fr;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) bo[j][s2] = BM * 128 + r * 128 + 16 * ((4 * s2 + fq) ^ swz(r));
  }

#pragma unroll
  for (int t = 0; t < S - 1; ++t) issue(t);
  if constexpr (ISSUE == 3) {
    mfma::pingpong_loop<S, FM, FN, LPW, STAGE>(dyn_lds, issue, ao, bo, acc, nk, wm);
  } else
  for (int t = 0; t < nk; ++t) {
    // this wave's copies of tile t are done; the barrier makes everyone's
    // visible and frees the stage read in step t - 1 for tile t + S - 1
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((S - 2) * LPW));
    __builtin_amdgcn_s_barrier();
    if constexpr (ISSUE == 0) issue(t + S - 1);
    const uint8_t* st = dyn_lds + (t % S) * STAGE;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      bf16x8 a[FM], b[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) a[i] = *(const bf16x8*)(st + ao[i][s2]);
#pragma unroll
      for (int j = 0; j < FN; ++j) b[j] = *(const bf16x8*)(st + bo[j][s2]);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
      if constexpr (ISSUE == 1)
        if (s2 == 0) issue(t + S - 1);
    }
    if constexpr (ISSUE == 2) issue(t + S - 1);
  }

  // Output through LDS: the accumulators (lane holds column lane & 15, rows
  // 4 (lane >> 4) + e of each 16 x 16 block) go to a row-major tile (rows
  // padded to BN + 4 floats), then whole rows leave with 16-byte stores.
  constexpr int OLD = BN + 4;
  static_assert(BM * OLD * 4 <= S * STAGE, "output tile must fit the stages");
  float* so = (float*)dyn_lds;
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();   // every wave is done with the stages
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        so[(wm * WM + i * 16 + fq * 4 + e) * OLD + wn * WN + j * 16 + fr] = acc[i][j][e];
  __syncthreads();
  float* out = sout + (int64_t)ks * out_kstride;
  for (int q = threadIdx.x; q < BM * BN / 4; q += kThreads) {
    const int r = q / (BN / 4), c = (q % (BN / 4)) * 4;
    const int m = m0 + r, n = n0 + c;
    if (m < M && n < N) {   // N % 4 == 0: a group of 4 is all in or all out
      f32x4 v = *(const f32x4*)&so[r * OLD + c];
      if (gate)
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = apply_gate(v[e], gate);
      f32x4* dst = (f32x4*)(out + (int64_t)phys(m) * ldo + n);
      if (STREAM)
        __builtin_nontemporal_store(v, dst);
      else
        *dst = v;
    }
  }
}

// The tile of work-group `bid` of a grid of `nb` over the segments of Pb.
template <int BM, int BN, int S, int NW, int ISSUE, bool STREAM>
__device__ __forceinline__ void run_tile(const Problem& Pb, int bid, int nb) {

  // Every kernel-argument scalar is read up front and every choice below is
  // a select, not a branch: the scalar loads then go out together instead
  // of one dependent round trip each.
  const int ksplit = Pb.ksplit, K = Pb.K;
  const int full = nb / kXcds * kXcds;
  const int bx = bid < full ? (bid % kXcds) * (full / kXcds) + bid / kXcds : bid;
  const int tb1 = Pb.tile_begin[1], tb2 = Pb.tile_begin[2], tb3 = Pb.tile_begin[3];
  asm volatile("" ::"s"(ksplit), "s"(K), "s"(tb1), "s"(tb2), "s"(tb3), "s"(nb));   // one round trip
  const int tile_ = ksplit == 1 ? bx : bid / ksplit;
  // tile_begin[i] for i >= nseg is the tile total
  const int si = (tile_ >= tb1 ? 1 : 0) + (tile_ >= tb2 ? 1 : 0) + (tile_ >= tb3 ? 1 : 0);
  static_assert(kMaxSeg == 4, "segment index select");
  const GemmSeg& S_ = Pb.s[si];
  const uint16_t* sx = S_.x;
  const int32_t* sgather = S_.gather;
  const int x_rows = S_.x_rows, ldx = S_.ldx, M = S_.M, N = S_.N, sn0 = S_.n0;
  const uint16_t *w0 = S_.w0, *w1 = S_.w1;
  const int tiles_n = S_.tiles_n;
  float* const sout = S_.out;
  const int64_t ldo = S_.ldo, out_kstride = S_.out_kstride;
  const int gate = S_.gate;
  const int grows = S_.grp_rows, gstride = S_.grp_stride;
  const int tbegin = Pb.tile_begin[si];
  asm volatile("" ::"s"(sx), "s"(sgather), "s"(x_rows), "s"(ldx), "s"(M), "s"(N), "s"(sn0), "s"(w0),
               "s"(w1), "s"(tiles_n), "s"(sout), "s"(ldo), "s"(out_kstride), "s"(gate), "s"(grows),
               "s"(gstride), "s"(tbegin), "s"(ksplit), "s"(K));   // one round trip
  const int tile = ksplit == 1 ? bx : bid / ksplit;
  const int ks = ksplit == 1 ? 0 : bid % ksplit;
  const int local = tile - tbegin;
  const int m0 = (local / tiles_n) * BM, n0 = (local % tiles_n) * BN;
  tile_core<BM, BN, S, NW, ISSUE, STREAM>(sx, sgather, x_rows, ldx, M, N, sn0, w0, w1, sout, ldo, out_kstride, gate, grows,
                                  gstride, K, m0, n0, ks, ksplit);
}

// One dense problem (no gather, no row map, no gate, one weight matrix, x
// holding exactly the M rows, K slices of [M, ldo] one after another):
// 48 bytes of arguments, which the command processor preloads into SGPRs
// when the kernel takes them as separate scalars (it preloads 56 bytes), so
// the work-group starts without a scalar load -- the conv's tap GEMM and H;
// with the 464-byte Problem, which is loaded from memory, the conv GEMM's
// prologue spent about 2,000 cycles on its arguments.
struct DenseProblem {
  const uint16_t* x;    // [M, K] rows, ldx elements apart
  const uint16_t* w;    // [N, K]
  float* out;           // out[m * ldo + n] (+ slice * M * ldo)
  int M, N, K, ksplit;
  int ldx, ldo;
};

template <int BM, int BN, int S, int NW, int ISSUE, bool STREAM>
__device__ __forceinline__ void run_tile_dense(const DenseProblem& D, int bid) {
  const int ksplit = D.ksplit;
  const int tiles_n = (D.N + BN - 1) / BN;
  const int nb = ((D.M + BM - 1) / BM) * tiles_n * ksplit;   // the grid
  const int full = nb / kXcds * kXcds;
  const int bx = bid < full ? (bid % kXcds) * (full / kXcds) + bid / kXcds : bid;
  // With a K split, bx enumerates (N-block, K slice) pairs with the M-block
  // fastest, so an XCD's work-groups (consecutive bx) cover a few slices of
  // one N-block for every M-block.  Against slice-fastest work-group order
  // (bx = bid): the batch-32 / block-16 step 0.4624 -> 0.4567 ms, the
  // stress cycle 826 -> 818 us; pairing N-blocks of one slice instead (the
  // XCD's work-groups then read the same K offsets at once) took 0.4731.
  const int tiles_m = (D.M + BM - 1) / BM;
  const int pair = bx / tiles_m, mb = bx % tiles_m;
  const int tile = ksplit == 1 ? bx : mb * tiles_n + pair / ksplit;
  const int ks = ksplit == 1 ? 0 : pair % ksplit;
  const int m0 = (tile / tiles_n) * BM, n0 = (tile % tiles_n) * BN;
  tile_core<BM, BN, S, NW, ISSUE, STREAM>(D.x, nullptr, D.M, D.ldx, D.M, D.N, D.N, D.w, D.w, D.out, D.ldo,
                                  (int64_t)D.M * D.ldo, 0, 0, 1, D.K, m0, n0, ks, ksplit);
}

// Fill P for up to kMaxSeg problems (hipErrorInvalidValue for shapes the
// kernel does not take), and raise a kernel's dynamic-LDS limit once.
hipError_t make_problem(const GemmSeg* segs, int nseg, int K, int ksplit, int bm, int bn, Problem& P,
                        int& tiles);
hipError_t allow_lds(const void* fn, int bytes, bool& done);

}  // namespace gemm
}  // namespace df2

// lmhead.hip -- drafter logits through the shared LM head, fused with the
// per-row top-K, so that the logits never reach memory.
//
// The drafter reuses the target's embedding and LM head ("大模型推理，加速王者：
// DFlash", paragraph before the three-step pipeline), and the selector takes
// its top-k candidates from that dense head ("DFlash 2 讓 Qwen3.8-27B 快了兩倍",
// 坑 2-4; the K = 16 kept per draft position: "DFlash 2: Keep Drafting
// Parallel", sections "The right tokens are already there" and "A
// lightweight path selector").  For rows r (draft positions, h [M, d]) and
// tokens v (E [V, d]):  z[r, v] = <h_r, E_v>  (bf16 products, fp32 sums),
// then the K best per row by (value desc, index asc).
//
// Two launches:
//  1. lmhead_topk_kernel: the product on the matrix cores, 256 x 128 or
//     128 x 128 tiles (rows of h x tokens; 256 rows wherever they add no
//     padding), K-tiles of 64 staged through 3 or 4 LDS stages by direct
//     buffer-to-LDS loads (mfma_tile.h), 8 waves.  A work-group owns one
//     row block and a contiguous range of 128-token blocks; after each token
//     block the fp32 tile goes through LDS, and thread (row, q) of the row's
//     Q = 2 or 4 threads folds columns q, q + Q, ... of its row into a
//     running best-16 list
//     held in registers (a sorted insertion, taken only by the few values
//     at or above the row's current threshold, found with one fp32 compare
//     each).  At the end the Q lists of a row are ranked against
//     each other and the row's 16 best keys of the range are written out.
//     The work-groups that share a token range (one per row block) run on
//     one XCD, one after the other in dispatch order, so that the token
//     block is fetched from memory once for all of them.
//  2. lmhead_merge_kernel: one work-group per row merges the ranges' lists:
//     the largest of the lists' 16th keys bounds the row's 16th best from
//     below (that list holds 16 keys at least as large), and the keys that
//     reach it are ranked against each other.
// Keys are the 64-bit (value, index) codes of df2_device.h: the result is
// the same whatever the order in which tokens are seen.
#include "df2_device.h"
#include "df2_internal.h"
#include "mfma_tile.h"

namespace df2 {

extern __shared__ __attribute__((aligned(16))) uint8_t dyn_lds[];

namespace {

using mfma::BK;
using mfma::load_lds16;
using mfma::swz;
using mfma::vmcnt_imm;

// Work-group tile: BM rows of h x 128 tokens, 8 waves, K-tiles of 64 through
// LDS stages.  BM = 128: waves 2 x 4 (64 x 32 each), 4 stages (128 KB), four
// threads per row in the epilogues; BM = 256: waves 4 x 2 (64 x 64 each: half
// the fragment bytes per MFMA, and a token block's rows are fetched by half
// as many work-groups), 3 stages (144 KB), two threads per row; BM = 64 (a
// few rows: the head is streamed from memory, and the padding rows' MFMAs
// halve): waves 2 x 4 (32 x 32 each), 6 stages (144 KB: five K-tiles of
// copies in flight), eight threads per row.
constexpr int kBN = 128, kNW = 8;
constexpr int kThreads = kNW * 64;
constexpr int kOld = kBN + 4;   // padded row of the fp32 tile
constexpr int kMaxRanges = 256;
static_assert(kBN == kHeadBlock, "statistics are kept per token block");
template <int BM>
struct HeadTile {
  static constexpr int kBM = BM;
  static constexpr int kWcol = BM == 256 ? 2 : 4;   // waves along the tokens
  static constexpr int kWM = kBM / (kNW / kWcol), kWN = kBN / kWcol;
  static constexpr int kFM = kWM / 16, kFN = kWN / 16;
  static constexpr int kALD = kBM / (8 * kNW), kBLD = kBN / (8 * kNW);   // loads per wave per stage
  static constexpr int kLPW = kALD + kBLD;
  static constexpr int kStage = (kBM + kBN) * BK * 2;   // bytes
  static constexpr int kS = BM == 64 ? 6 : (BM == 128 ? 4 : 3);
  static constexpr int kLds = kS * kStage;
  static constexpr int kQ = kThreads / kBM;   // threads per row
  static constexpr int kCpt = 16 / kQ;        // candidates (statistics) and output keys per thread
  static_assert(BM == 64 || BM == 128 || BM == 256, "row tile");
  static_assert(kBM * kOld * 4 <= kLds, "fp32 tile fits the stages");
  static_assert(kBM * kQ * 16 * 8 + kBM * 16 * 8 <= kLds, "the rows' lists and results fit the stages");
  static_assert(kQ == 2 || kQ == 4 || kQ == 8, "threads per row");
};

// Insert key x into the list l[0] > l[1] > ... > l[15] (0 = empty) when it
// is larger than l[15]: every entry moves down one place past x.
__device__ __forceinline__ void insert16(uint64_t (&l)[16], uint64_t x) {
#pragma unroll
  for (int i = 15; i > 0; --i) {
    const uint64_t up = l[i - 1];
    l[i] = x > up ? up : (x > l[i] ? x : l[i]);
  }
  l[0] = x > l[0] ? x : l[0];
}

// grid: mblocks * nranges work-groups of kThreads; dynamic LDS kLds.
// part[(row * nranges + range) * KEEP + i]: the i-th best key of the range
// (KEEP = 16: the drafter's top-16; KEEP = 1: the target's argmax).
// KEEP = 0 (statistics for rejection verification): per row and 128-token
// block the online-softmax partial hs.stats, and the logits of the row's
// candidates (hs.zc) and drafted token (hs.zx) as their blocks go by.
template <int KEEP, int BM>
__global__ __launch_bounds__(kThreads) void lmhead_topk_kernel(
    const uint16_t* __restrict__ h, int M, const uint16_t* __restrict__ emb, int64_t vocab, int K,
    int mblocks, int nranges, int nblocks, int xcd_groups, uint64_t* __restrict__ part, HeadStats hs) {
  using TT = HeadTile<BM>;
  constexpr int kBM = TT::kBM, kWcol = TT::kWcol, kWM = TT::kWM, kWN = TT::kWN, kFM = TT::kFM, kFN = TT::kFN;
  constexpr int kALD = TT::kALD, kBLD = TT::kBLD, kLPW = TT::kLPW, kStage = TT::kStage, kS = TT::kS;
  constexpr int kQ = TT::kQ, kCpt = TT::kCpt;
  // one bit per column of a thread's share of a token block
  using Mask = typename std::conditional<(kBN / kQ > 32), uint64_t, uint32_t>::type;
  const int bid = blockIdx.x;
  int mb, nr;
  if (xcd_groups) {   // nranges % 8 == 0: the row blocks of a token range share an XCD
    const int x = bid % 8, q = bid / 8;
    mb = q % mblocks;
    nr = (q / mblocks) * 8 + x;
  } else {
    mb = bid % mblocks;
    nr = bid / mblocks;
  }
  const int nb0 = (int)((int64_t)nr * nblocks / nranges), nb1 = (int)((int64_t)(nr + 1) * nblocks / nranges);
  const int m0 = mb * kBM;
  const int wave = wave_id(), lane = lane_id();
  const int wm = wave / kWcol, wn = wave % kWcol;
  const int nkt = K / BK;
  const int sub = lane >> 3, slot = lane & 7;
  const int fr = lane & 15, fq = lane >> 4;
  // h rows: one buffer resource for the row block (rows past M read zeros)
  const int hrows = M - m0 < kBM ? M - m0 : kBM;
  const __amdgpu_buffer_rsrc_t hres =
      __builtin_amdgcn_make_buffer_rsrc((void*)(h + (int64_t)m0 * K), 0, hrows * K * 2, kBufferWord3);
  const uint32_t kOut = 0xFFFFFFF0u - (uint32_t)K * 2u;   // beyond every buffer for the whole K walk
  uint32_t xo[kALD], wo[kBLD];
#pragma unroll
  for (int a = 0; a < kALD; ++a) {
    const int row = 8 * (wave + kNW * a) + sub;
    xo[a] = row < hrows ? (uint32_t)((row * K + ((slot ^ swz(row)) * 8)) * 2) : kOut;
  }
  // fragment byte offsets inside a stage (rows fixed per lane, chunk 4 s + fq)
  int ao[kFM][2], bo[kFN][2];
#pragma unroll
  for (int i = 0; i < kFM; ++i) {
    const int r = wm * kWM + i * 16 + fr;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) ao[i][s2] = r * 128 + 16 * ((4 * s2 + fq) ^ swz(r));
  }
#pragma unroll
  for (int j = 0; j < kFN; ++j) {
    const int r = wn * kWN + j * 16 + fr;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) bo[j][s2] = kBM * 128 + r * 128 + 16 * ((4 * s2 + fq) ^ swz(r));
  }
  // the running best KEEP keys of this thread: row tid / 4, columns
  // tid % 4 + 4 j
  static_assert(KEEP == 16 || KEEP == 1 || KEEP == 0, "best-16 lists, the argmax, or statistics");
  const int my_row = threadIdx.x / kQ, my_q = threadIdx.x % kQ;
  uint64_t best[KEEP > 0 ? KEEP : 1];
#pragma unroll
  for (int i = 0; i < (KEEP > 0 ? KEEP : 1); ++i) best[i] = 0ull;
  float* tile = (float*)dyn_lds;
  // statistics mode: this thread's 16 / Q candidates of its row (ranks
  // q 16 / Q onwards) and, for q = 0, the drafted token
  int32_t cid[kCpt];
#pragma unroll
  for (int i = 0; i < kCpt; ++i) cid[i] = -1;
  int32_t xt = -1;
  if constexpr (KEEP == 0) {
    const int r = m0 + my_row, b = r / (hs.T + 1), t = r % (hs.T + 1);
    if (r < M && t < hs.T) {
#pragma unroll
      for (int i = 0; i < kCpt; ++i) {
        const int k = my_q * kCpt + i;
        if (k < hs.K) cid[i] = hs.cand[((int64_t)b * hs.T + t) * hs.K + k];
      }
      if (my_q == 0) xt = hs.xtok[(int64_t)b * hs.T + t];
    }
  }

  for (int nb = nb0; nb < nb1; ++nb) {
    const int64_t n0 = (int64_t)nb * kBN;
    const int wrows = vocab - n0 < kBN ? (int)(vocab - n0) : kBN;
    const __amdgpu_buffer_rsrc_t eres =
        __builtin_amdgcn_make_buffer_rsrc((void*)(emb + n0 * K), 0, wrows * K * 2, kBufferWord3);
#pragma unroll
    for (int b = 0; b < kBLD; ++b) {
      const int row = 8 * (wave + kNW * b) + sub;
      wo[b] = row < wrows ? (uint32_t)((row * K + ((slot ^ swz(row)) * 8)) * 2) : kOut;
    }
    auto issue = [&](int t) {
      const bool in = t < nkt;
      uint8_t* sb = dyn_lds + (t % kS) * kStage;
      const int so = __builtin_amdgcn_readfirstlane(in ? t * BK * 2 : 0);
      const uint32_t dx = in ? 0u : kOut;   // past the end: reads nothing
#pragma unroll
      for (int a = 0; a < kALD; ++a) load_lds16(hres, sb + (wave + kNW * a) * 8 * 128, xo[a] | dx, so);
#pragma unroll
      for (int b = 0; b < kBLD; ++b)
        load_lds16(eres, sb + kBM * 128 + (wave + kNW * b) * 8 * 128, wo[b] | dx, so);
    };
    f32x4 acc[kFM][kFN];
#pragma unroll
    for (int i = 0; i < kFM; ++i)
#pragma unroll
      for (int j = 0; j < kFN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < kS - 1; ++t) issue(t);
    // 256-row tiles: the waves in two alternating groups (mfma_tile.h; 2 %
    // faster here, no gain with 128-row tiles)
    if constexpr (BM == 256) {
      mfma::pingpong_loop<kS, kFM, kFN, kLPW, kStage>(dyn_lds, issue, ao, bo, acc, nkt, wave / 4);
    } else
    for (int t = 0; t < nkt; ++t) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm((kS - 2) * kLPW));
      __builtin_amdgcn_s_barrier();
      const uint8_t* st = dyn_lds + (t % kS) * kStage;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        bf16x8 a[kFM], b[kFN];
#pragma unroll
        for (int i = 0; i < kFM; ++i) a[i] = *(const bf16x8*)(st + ao[i][s2]);
#pragma unroll
        for (int j = 0; j < kFN; ++j) b[j] = *(const bf16x8*)(st + bo[j][s2]);
#pragma unroll
        for (int i = 0; i < kFM; ++i)
#pragma unroll
          for (int j = 0; j < kFN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
      }
      // next copies behind the MFMAs, into the stage every wave left before
      // this step's barrier (as in gemm_tile.h)
      issue(t + kS - 1);
    }
    // the fp32 tile through LDS (lane holds column lane & 15, rows
    // 4 (lane >> 4) + e of each 16 x 16 block), then each thread folds its
    // columns of its row into its list
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();   // every wave is done with the stages
#pragma unroll
    for (int i = 0; i < kFM; ++i)
#pragma unroll
      for (int j = 0; j < kFN; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          tile[(wm * kWM + i * 16 + fq * 4 + e) * kOld + wn * kWN + j * 16 + fr] = acc[i][j][e];
    __syncthreads();
    // The row's threshold: the largest of its threads' 16th keys (the
    // row has 16 keys at least that large, so no key at or below it can be
    // among its 16 best).  One fp32 compare per value against the
    // threshold's value marks the few that may pass; only those are made
    // into keys and inserted (the wave runs the insertion loop as often as
    // its busiest lane needs, not once per value).
    const float* trow = tile + my_row * kOld;
    // columns past the vocabulary are not tokens; rows past M (zeros) are
    // not rows: their threads skip the fold
    const int ncols = m0 + my_row < M ? wrows : 0;
    if constexpr (KEEP == 0) {
      // the block's online-softmax partial of this row: each thread over its
      // columns, then the row's threads combined (symmetrically: all of
      // them hold the same result)
      float v[kBN / kQ];
#pragma unroll
      for (int j = 0; j < kBN / kQ; ++j) v[j] = trow[my_q + kQ * j];
      uint64_t mk = 0ull;
#pragma unroll
      for (int j = 0; j < kBN / kQ; ++j) {
        const int c = my_q + kQ * j;
        const uint64_t key = make_key(v[j], (uint32_t)(n0 + c));
        if (c < ncols && v[j] == v[j] && key > mk) mk = key;
      }
      float sum = 0.f;
      if (mk) {
        const float m = key_value(mk);
#pragma unroll
        for (int j = 0; j < kBN / kQ; ++j)
          if (my_q + kQ * j < ncols && v[j] == v[j]) sum += v[j] == m ? 1.f : exp2f((v[j] - m) * hs.c);
      }
#pragma unroll
      for (int msk = 1; msk < kQ; msk <<= 1) {
        const uint64_t k2 = shfl_xor_u64(mk, msk);
        const float s2 = __shfl_xor(sum, msk);
        uint64_t ka = mk < k2 ? mk : k2, kb = mk < k2 ? k2 : mk;
        float sa = mk < k2 ? sum : s2, sb = mk < k2 ? s2 : sum;
        combine_part(kb, sb, ka, sa, hs.c);
        mk = kb;
        sum = sb;
      }
      const int r = m0 + my_row;
      if (my_q == 0 && r < M) {
        BlockStat bs;
        bs.key = mk;
        bs.s = sum;
        bs.pad = 0.f;
        hs.stats[(int64_t)r * nblocks + nb] = bs;
      }
#pragma unroll
      for (int i = 0; i < kCpt; ++i)
        if (cid[i] >= n0 && cid[i] < n0 + ncols) hs.zc[(int64_t)r * hs.K + my_q * kCpt + i] = trow[cid[i] - n0];
      if (xt >= n0 && xt < n0 + ncols) hs.zx[r] = trow[xt - n0];
      __syncthreads();   // the tile is read before the next block's stages overwrite it
      continue;
    }
    uint64_t thr = best[KEEP > 0 ? KEEP - 1 : 0];
#pragma unroll
    for (int msk = 1; msk < kQ; msk <<= 1) {
      const uint64_t o = shfl_xor_u64(thr, msk);
      thr = o > thr ? o : thr;
    }
    const float tv = thr ? key_value(thr) : -INFINITY;
    float v[kBN / kQ];
#pragma unroll
    for (int j = 0; j < kBN / kQ; ++j) v[j] = trow[my_q + kQ * j];
    Mask mask = 0;
#pragma unroll
    for (int j = 0; j < kBN / kQ; ++j)
      mask |= (my_q + kQ * j < ncols && v[j] >= tv) ? ((Mask)1 << j) : (Mask)0;   // NaN never passes
    while (mask) {
      const int j = sizeof(Mask) == 8 ? __builtin_ctzll((uint64_t)mask) : __builtin_ctz((uint32_t)mask);
      mask &= mask - 1;
      const int c = my_q + kQ * j;
      const uint64_t key = make_key(trow[c], (uint32_t)(n0 + c));
      if constexpr (KEEP == 16) {
        if (key > thr && key > best[15]) insert16(best, key);
      } else {
        best[0] = key > best[0] ? key : best[0];
      }
    }
    __syncthreads();   // the tile is read before the next block's stages overwrite it
  }

  if constexpr (KEEP == 0) return;
  if constexpr (KEEP == 1) {
    // the row's argmax key of the range: the largest of its threads'
    uint64_t m = best[0];
#pragma unroll
    for (int msk = 1; msk < kQ; msk <<= 1) {
      const uint64_t o = shfl_xor_u64(m, msk);
      m = o > m ? o : m;
    }
    if (my_q == 0 && m0 + my_row < M) part[(int64_t)(m0 + my_row) * nranges + nr] = m;
    return;
  }
  // the Q lists of each row, ranked against each other
  uint64_t* lists = (uint64_t*)dyn_lds;   // [kBM][kQ * 16]
#pragma unroll
  for (int i = 0; i < KEEP; ++i) lists[my_row * (kQ * 16) + my_q * 16 + i] = best[i];
  __syncthreads();
  uint64_t* out16 = lists + kBM * kQ * 16;   // [kBM][16], after the lists
  if (my_q == 0)
#pragma unroll
    for (int i = 0; i < 16; ++i) out16[my_row * 16 + i] = 0ull;
  __syncthreads();
  const uint64_t* rl = lists + my_row * (kQ * 16);
#pragma unroll
  for (int i = 0; i < KEEP; ++i) {   // unrolled: best[] stays in registers
    const uint64_t key = best[i];
    if (key == 0ull) continue;
    int rank = 0;
    for (int j = 0; j < kQ * 16; ++j) rank += rl[j] > key ? 1 : 0;
    if (rank < 16) out16[my_row * 16 + rank] = key;
  }
  __syncthreads();
  // rows of the block that exist: 16 keys each, kQ threads per row
  if (m0 + my_row < M) {
    uint64_t* dst = part + ((int64_t)(m0 + my_row) * nranges + nr) * 16;
#pragma unroll
    for (int i = 0; i < kCpt; ++i) dst[my_q * kCpt + i] = out16[my_row * 16 + my_q * kCpt + i];
  }
}

// One work-group per row: the 16 best of nranges lists of 16 (each best
// first, empty slots 0).
constexpr int kMergeThreads = 256;
__global__ __launch_bounds__(kMergeThreads) void lmhead_merge_kernel(const uint64_t* __restrict__ part,
                                                                      int nranges, int k,
                                                                      int32_t* __restrict__ out_idx,
                                                                      float* __restrict__ out_val) {
  __shared__ uint64_t surv[kMaxRanges * 16];
  __shared__ uint64_t heads[kMaxRanges + 16];
  __shared__ uint64_t sbound[kMergeThreads / 64];
  __shared__ uint64_t sb2;
  __shared__ int nsurv;
  __shared__ uint64_t res[16];
  const int row = blockIdx.x, tid = threadIdx.x;
  const uint64_t* p = part + (int64_t)row * nranges * 16;
  // Two lower bounds on the row's 16th best key: the largest of the lists'
  // 16th keys (that list holds 16 keys at least as large), and the 16th
  // largest among the first j keys of every list (j = ceil(16 / nranges):
  // at least 16 distinct keys of the row).  With many short ranges the
  // second is the tight one (the 16th best of the ranges' best keys).
  uint64_t b = 0ull;
  for (int l = tid; l < nranges; l += kMergeThreads) b = p[l * 16 + 15] > b ? p[l * 16 + 15] : b;
  b = wave_max_u64(b);
  if (lane_id() == 0) sbound[tid / 64] = b;
  const int j = (16 + nranges - 1) / nranges;   // nranges * j <= kMaxRanges + 15
  const int nh = nranges * j;
  for (int s = tid; s < nh; s += kMergeThreads) heads[s] = p[(s / j) * 16 + s % j];
  if (tid == 0) {
    nsurv = 0;
    sb2 = 0ull;
  }
  if (tid < 16) res[tid] = 0ull;
  __syncthreads();
  for (int s = tid; s < nh; s += kMergeThreads) {
    const uint64_t key = heads[s];
    int rank = 0;
    for (int q = 0; q < nh; ++q) rank += heads[q] > key ? 1 : 0;
    if (key != 0ull && rank == 15) sb2 = key;   // keys are distinct: one writer
  }
  __syncthreads();
  uint64_t bound = sb2;
#pragma unroll
  for (int w = 0; w < kMergeThreads / 64; ++w) bound = sbound[w] > bound ? sbound[w] : bound;
  for (int s = tid; s < nranges * 16; s += kMergeThreads) {
    const uint64_t key = p[s];
    if (key != 0ull && key >= bound) surv[atomicAdd(&nsurv, 1)] = key;
  }
  __syncthreads();
  const int ns = nsurv;
  for (int s = tid; s < ns; s += kMergeThreads) {
    const uint64_t key = surv[s];
    int rank = 0;
    for (int j = 0; j < ns; ++j) rank += surv[j] > key ? 1 : 0;
    if (rank < 16) res[rank] = key;
  }
  __syncthreads();
  if (tid < k) {
    const uint64_t key = res[tid];
    out_idx[(int64_t)row * k + tid] = (int32_t)key_index(key);
    out_val[(int64_t)row * k + tid] = key_value(key);
  }
}

// Greedy verification from the argmax keys: one work-group of four waves
// per request; wave w takes rows t = w, w + 4, ... (t <= T), its lanes the
// row's ranges (all their keys requested before the maximum is taken), and
// the row's argmax goes to LDS; then wave 0 finds n = the longest prefix on
// which the drafted tokens equal the argmax and emits the n accepted drafts,
// the argmax at n, then -1.
constexpr int kFinalThreads = 256;
__global__ __launch_bounds__(kFinalThreads) void greedy_head_final_kernel(const uint64_t* __restrict__ part,
                                                                          int nranges,
                                                                          const int32_t* __restrict__ path_tok,
                                                                          int T, int32_t* __restrict__ accept_len,
                                                                          int32_t* __restrict__ out_tok) {
  __shared__ uint64_t sy[64];
  const int b = blockIdx.x, lane = lane_id(), wave = threadIdx.x / kWave;
  constexpr int kPer = kMaxRanges / kWave;   // keys per lane per row (nranges <= kMaxRanges)
  for (int t = wave; t <= T; t += kFinalThreads / kWave) {
    const uint64_t* p = part + ((int64_t)b * (T + 1) + t) * nranges;
    uint64_t k[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int r = lane + i * kWave;
      k[i] = r < nranges ? p[r] : 0ull;
    }
    uint64_t m = 0ull;
#pragma unroll
    for (int i = 0; i < kPer; ++i) m = k[i] > m ? k[i] : m;
    m = wave_max_u64(m);
    if (lane == 0) sy[t] = m;
  }
  __syncthreads();
  if (wave != 0) return;
  const int32_t y = lane <= T ? (int32_t)key_index(sy[lane]) : -1;
  const int32_t x = lane < T ? path_tok[(int64_t)b * T + lane] : -1;
  const uint64_t miss = ballot(lane < T && x != y);
  const int n = miss ? __ffsll((unsigned long long)miss) - 1 : T;
  if (lane == 0) accept_len[b] = n;
  if (lane <= T) out_tok[(int64_t)b * (T + 1) + lane] = lane < n ? x : (lane == n ? y : -1);
}

// Launch lmhead_topk_kernel<KEEP, BM> over the plan's grid (its dynamic-LDS
// limit raised on first use).
template <int KEEP, int BM>
hipError_t launch_head_tiles(const void* h, int M, const void* emb, int64_t vocab, int d, const LmHeadPlan& plan,
                             uint64_t* part, const HeadStats& hs, const char* tag, hipStream_t stream) {
  constexpr int kLds = HeadTile<BM>::kLds;
  static bool lds_set = false;
  if (!lds_set) {
    hipError_t e = hipFuncSetAttribute((const void*)lmhead_topk_kernel<KEEP, BM>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
    if (e != hipSuccess) return e;
    lds_set = true;
  }
  ProfileScope ps(tag, stream);
  return launch(lmhead_topk_kernel<KEEP, BM>, dim3((unsigned)(plan.mblocks * plan.nranges)), dim3(kThreads), kLds,
                stream, ps, (const uint16_t*)h, M, (const uint16_t*)emb, vocab, d, plan.mblocks, plan.nranges,
                plan.nblocks, plan.xcd_groups, part, hs);
}

template <int KEEP>
hipError_t launch_head(const void* h, int M, const void* emb, int64_t vocab, int d, const LmHeadPlan& plan,
                       uint64_t* part, const HeadStats& hs, const char* tag, hipStream_t stream) {
  if (plan.bm == 64) return launch_head_tiles<KEEP, 64>(h, M, emb, vocab, d, plan, part, hs, tag, stream);
  return plan.bm == 256 ? launch_head_tiles<KEEP, 256>(h, M, emb, vocab, d, plan, part, hs, tag, stream)
                        : launch_head_tiles<KEEP, 128>(h, M, emb, vocab, d, plan, part, hs, tag, stream);
}

}  // namespace

LmHeadPlan lmhead_plan(int M, int64_t vocab, int d, int keep) {
  (void)d;
  LmHeadPlan p;
  // 64-row tiles up to 64 rows; 256-row tiles where they add no padding rows
  // over 128-row ones (and from 1,024 rows on, where the extra padding is at
  // most 1/8); else 128
  const int64_t pad128 = ((int64_t)M + 127) / 128 * 128, pad256 = ((int64_t)M + 255) / 256 * 256;
  p.bm = M <= 64 ? 64 : ((M > 128 && pad256 == pad128) || M >= 1024 ? 256 : 128);
  p.mblocks = (M + p.bm - 1) / p.bm;
  p.nblocks = (int)((vocab + kBN - 1) / kBN);
  // about one work-group per CU (each holds 128 or 144 KB of LDS and 8 waves)
  int nr = 256 / (p.mblocks > 0 ? p.mblocks : 1);
  if (nr < 1) nr = 1;
  if (nr > p.nblocks) nr = p.nblocks;
  if (nr > kMaxRanges) nr = kMaxRanges;
  if (nr >= 8) nr = nr / 8 * 8;
  p.nranges = nr;
  p.xcd_groups = nr % 8 == 0 ? 1 : 0;
  p.ws_bytes = align256((size_t)M * (size_t)nr * (size_t)keep * sizeof(uint64_t));
  return p;
}

hipError_t launch_lmhead_topk(const void* h, const void* emb, int64_t vocab, int M, int d, int k,
                              int32_t* out_idx, float* out_val, void* ws, const LmHeadPlan& plan,
                              hipStream_t stream) {
  if (M == 0) return hipSuccess;
  uint64_t* part = (uint64_t*)ws;
  DF2_TRY(launch_head<16>(h, M, emb, vocab, d, plan, part, HeadStats{}, "lmhead_topk", stream));
  ProfileScope ps("lmhead_merge", stream);
  DF2_TRY(launch(lmhead_merge_kernel, dim3((unsigned)M), dim3(kMergeThreads), 0, stream, ps, part,
                 plan.nranges, k, out_idx, out_val));
  return hipGetLastError();
}

hipError_t launch_verify_greedy_head(const void* h, const void* emb, int64_t vocab, int d,
                                    const int32_t* path_tok, int B, int T, int32_t* accept_len,
                                    int32_t* out_tok, void* ws, const LmHeadPlan& plan, hipStream_t stream) {
  if (B == 0) return hipSuccess;
  const int M = B * (T + 1);
  uint64_t* part = (uint64_t*)ws;
  DF2_TRY(launch_head<1>(h, M, emb, vocab, d, plan, part, HeadStats{}, "head_argmax", stream));
  ProfileScope ps("greedy_head_final", stream);
  DF2_TRY(launch(greedy_head_final_kernel, dim3((unsigned)B), dim3(kFinalThreads), 0, stream, ps, part, plan.nranges,
                 path_tok, T, accept_len, out_tok));
  return hipGetLastError();
}

hipError_t launch_head_stats(const void* h, const void* emb, int64_t vocab, int M, int d, const HeadStats& hs,
                             const LmHeadPlan& plan, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  DF2_TRY(launch_head<0>(h, M, emb, vocab, d, plan, (uint64_t*)nullptr, hs, "head_stats", stream));
  return hipGetLastError();
}

}  // namespace df2

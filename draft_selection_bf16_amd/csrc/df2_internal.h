// df2_internal.h -- host-side launchers of the draft-block kernels.
// Internal; the C ABI (api.hip) validates arguments and calls these.
#pragma once

#include <hip/hip_ext.h>
#include <tuple>
#include <utility>

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace df2 {

// Kernel timing hook (see dflash2_profile_start): a scope names the kernel
// tag of the launch it wraps; when that tag is armed and slots are left, the
// launch records a start and a stop event in its dispatch (the kernel's own
// duration, no stream-side overhead).
struct ProfileScope {
  ProfileScope(const char* tag, hipStream_t stream);
  bool on;
  hipEvent_t start, stop;
  void used();   // the events of this scope were recorded
};

// Launch `k` with arguments converted to its exact parameter types; timed
// through the scope's events when it is armed.
template <typename... P, typename... A>
inline hipError_t launch(void (*k)(P...), dim3 grid, dim3 block, unsigned shmem, hipStream_t stream,
                         ProfileScope& ps, A&&... a) {
  std::tuple<P...> vals(std::forward<A>(a)...);
  void* ptrs[sizeof...(P) > 0 ? sizeof...(P) : 1];
  std::apply([&](auto&... x) {
    int i = 0;
    ((ptrs[i++] = (void*)&x), ...);
  }, vals);
  if (ps.on) {
    hipError_t e = hipExtLaunchKernel((const void*)k, grid, block, ptrs, shmem, stream, ps.start, ps.stop, 0);
    if (e == hipSuccess) ps.used();
    return e;
  }
  return hipLaunchKernel((const void*)k, grid, block, ptrs, shmem, stream);
}

// Return a launch failure from the enclosing launcher.
#define DF2_TRY(call)                     \
  do {                                    \
    const hipError_t df2_e_ = (call);     \
    if (df2_e_ != hipSuccess) return df2_e_; \
  } while (0)

// Aligned sub-buffer carving of a caller workspace.
inline size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// ---- top-K -----------------------------------------------------------------
struct TopkPlan {
  int splits;       // work-groups per row
  int64_t chunk;    // elements per split (multiple of 64)
  int small;        // 1: the short-chunk kernel (chunk <= 8192)
  size_t ws_bytes;  // partial-key buffer
};
TopkPlan topk_plan(int64_t rows, int64_t vocab, int k);
hipError_t launch_topk(const void* logits, int dt, int64_t rows, int64_t vocab, int k,
                       int32_t* out_idx, float* out_val, void* ws, const TopkPlan& plan,
                       hipStream_t stream);

// ---- projection GEMM (bf16 MFMA, fp32 out) --------------------------------
struct GemmSeg {
  const uint16_t* x;      // bf16 rows
  const int32_t* gather;  // nullable: row ids into x (-> zero row if outside [0, x_rows))
  int64_t x_rows;         // number of rows x holds (bound for gather)
  int64_t ldx;            // elements between rows of x
  int M;                  // rows of the product
  const uint16_t* w0;     // W rows 0..n0-1
  const uint16_t* w1;     // W rows n0..N-1 (row n -> w1[n - n0])
  int n0;
  int N;                  // output columns (multiple of 16)
  float* out;             // out[m * ldo + n] (+ slice * out_kstride)
  int64_t ldo;
  int64_t out_kstride;    // elements between K-slice partial outputs
  int gate;               // 0 identity, 1 sigmoid (only when ksplit == 1)
  // grouped rows (grp_rows > 0): product row m is row
  // (m / grp_rows) * grp_stride + m % grp_rows of the gather list (or of x)
  // and of out -- the leading grp_rows of every group of grp_stride rows
  int grp_rows, grp_stride;
  int tiles_m, tiles_n;   // filled by the launcher
};
// Work-group tile BM x BN, LDS stages, waves per work-group.
struct GemmTiling {
  int bm, bn, stages, waves;
  int issue;   // copies of the next tiles issued 0 after the barrier, 1 mid-tile, 2 after the MFMAs;
               // 3: two alternating groups of four waves (waves = 8)
};
// out = gate(X W^T) for up to 4 segments in one launch; K = d (multiple of 64).
// Each segment needs n0 % bn == 0 or n0 >= N, and x_rows * ldx * 2 < 2^32.
// (bm, bn, stages, waves, issue) in {(64,128,3,4,1), (64,128,4,8,3), (128,128,4,8,3), (256,128,3,8,3)};
// K % 64 == 0 and
// 1 <= ksplit <= K / 64 (slices of K / 64 / ksplit K-tiles, rounded).
hipError_t launch_gemm(const GemmSeg* segs, int nseg, int K, int ksplit, const GemmTiling& t,
                       const char* tag, hipStream_t stream);

// ---- pair scores epilogue ---------------------------------------------------
// ab, a_last, h: `split` slices of partial products, kstrides floats apart;
// with split > 1 a reduce pass first sums them in slice order into slice 0
// (in place: the buffers are workspace); h ungated (the gate is applied
// after the sum).
hipError_t launch_pair_epilogue(float* ab, float* a_last, float* h, int split,
                                int64_t ab_k, int64_t alast_k, int64_t h_k, int gate,
                                const float* cand_val, int B, int T, int K, int r,
                                float* scores, hipStream_t stream);
// The same scores with A and B read from a per-token table tab [vocab, 2r]
// (A in columns 0..r-1, B in r..2r-1) by token id; h: `split` slices of
// ungated partial products, summed in slice order by the epilogue itself.
hipError_t launch_pair_epilogue_tab(const float* tab, int64_t vocab, const int32_t* cand_idx,
                                    const int32_t* last_tok, const float* h, int split, int64_t h_k, int gate,
                                    const float* cand_val, int B, int T, int K, int r, float* scores,
                                    hipStream_t stream);

// ---- path ------------------------------------------------------------------
hipError_t launch_path(const float* scores, const int32_t* cand_idx, int B, int T, int K, int mode,
                       float temperature, const uint64_t* seed_dev, int b0, int32_t* path_rank,
                       int32_t* path_tok, float* q, float* path_score, hipStream_t stream);

// ---- verification ------------------------------------------------------------
struct VerifyPlan {
  int splits;        // work-groups per target row in the streaming pass
  int64_t chunk;     // elements per split
  int rchunks;       // chunks of the residual scan per request
  int64_t rchunk;    // elements per residual chunk
  int fused;         // rejection: residual draw in one work-group per request over the chunks above
  size_t off_part;   // partial results [rows, splits] (8 bytes each)
  size_t off_dec;    // per-request decision record
  size_t off_rsum;   // residual chunk sums [B, rchunks]
  size_t ws_bytes;
};
VerifyPlan verify_plan(int B, int T, int64_t vocab);
hipError_t launch_verify_greedy(const void* z, int dt, int64_t vocab, const int32_t* path_tok,
                                int B, int T, int32_t* accept_len, int32_t* out_tok, void* ws,
                                const VerifyPlan& plan, hipStream_t stream);
hipError_t launch_verify_reject(const void* z, int dt, int64_t vocab, const int32_t* path_tok,
                                const int32_t* path_rank, const int32_t* cand_idx, const float* q,
                                int B, int T, int K, float temperature, const uint64_t* seed_dev, int b0,
                                int32_t* accept_len, int32_t* out_tok, void* ws,
                                const VerifyPlan& plan, hipStream_t stream);

// ---- two-tap dynamic conv ---------------------------------------------------
struct ConvPlan {
  int ksplit;
  GemmTiling tiling;
  size_t ws_bytes;    // the slices' partial products
};
ConvPlan conv_plan(int B, int L, int d, int group);
hipError_t launch_dynconv2(const void* x, const void* x_prev, const void* w, const float* base,
                           int B, int L, int d, int group, void* y, int y_dt, void* ws,
                           const ConvPlan& plan, hipStream_t stream);

// ---- drafter LM head fused with the top-K ----------------------------------
struct LmHeadPlan {
  int bm;           // rows of h per tile: 64, 128 or 256
  int mblocks;      // bm-row blocks of h
  int nblocks;      // 128-token blocks of the vocabulary
  int nranges;      // token ranges (work-groups per row block)
  int xcd_groups;   // nranges % 8 == 0: a range's row blocks run on one XCD
  size_t ws_bytes;  // per-range best keys [M, nranges, keep]
};
// keep = 16 (the drafter's top-16) or 1 (the target's argmax)
LmHeadPlan lmhead_plan(int M, int64_t vocab, int d, int keep);
// tokens per block of the fused LM-head kernels (the token side of a tile)
constexpr int kHeadBlock = 128;
// Online-softmax partial of one 128-token block of one row: key = the
// block's (max logit, lowest index), s = sum of exp2((z - max) c).
struct BlockStat {
  uint64_t key;
  float s;
  float pad;
};
// Statistics mode of the fused LM-head kernel (rejection verification):
// rows are (b, t) = (row / (T + 1), row % (T + 1)) of a [B, T+1] block.
struct HeadStats {
  float c;                 // log2(e) / temperature
  int T, K;
  const int32_t* cand;     // [B, T, K] candidates (t < T)
  const int32_t* xtok;     // [B, T] drafted tokens
  BlockStat* stats;        // [rows, nblocks]
  float* zc;               // [rows, K] logits of the candidates (t < T)
  float* zx;               // [rows] logit of the drafted token (t < T)
};
hipError_t launch_head_stats(const void* h, const void* emb, int64_t vocab, int M, int d, const HeadStats& hs,
                             const LmHeadPlan& plan, hipStream_t stream);
struct HeadRejectPlan {
  LmHeadPlan lm;
  size_t off_stats, off_rowst, off_zc, off_zx, off_dec, off_zblk;
  size_t ws_bytes;
};
HeadRejectPlan head_reject_plan(int B, int T, int64_t vocab, int d, int K);
hipError_t launch_verify_reject_head(const void* h, const void* emb, int64_t vocab, int d,
                                     const int32_t* path_tok, const int32_t* path_rank, const int32_t* cand_idx,
                                     const float* q, int B, int T, int K, float temperature,
                                     const uint64_t* seed_dev, int b0, int32_t* accept_len, int32_t* out_tok,
                                     void* ws, const HeadRejectPlan& plan, hipStream_t stream);
hipError_t launch_lmhead_topk(const void* h, const void* emb, int64_t vocab, int M, int d, int k,
                              int32_t* out_idx, float* out_val, void* ws, const LmHeadPlan& plan,
                              hipStream_t stream);
// greedy verification with the target logits computed from h [B, T+1, d]
// through the LM head (plan for M = B * (T + 1) rows, keep 1)
hipError_t launch_verify_greedy_head(const void* h, const void* emb, int64_t vocab, int d,
                                    const int32_t* path_tok, int B, int T, int32_t* accept_len,
                                    int32_t* out_tok, void* ws, const LmHeadPlan& plan, hipStream_t stream);

// ---- Philox words -----------------------------------------------------------
hipError_t launch_philox(const uint64_t* seed_dev, const int32_t* b, const int32_t* t, int n,
                         uint64_t* out, hipStream_t stream);

}  // namespace df2

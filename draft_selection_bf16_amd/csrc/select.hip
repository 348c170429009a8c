// select.hip -- the path selector after the projections: bilinear pair
// scores and the path through the K x K lattices.
//
// Pair score ("DFlash 2: Keep Drafting Parallel", section "A lightweight
// path selector", equation S_t(a,b) = U_t(b) + <A(a) (.) H(h_t), B(b)>):
// one work-group per (request, position); the predecessor rows A(a) (the
// candidates of position t-1, or the last verified token at t = 0) are
// scaled by the gate H_t once in LDS, then the K x K dot products with B(b)
// are taken register-blocked (each lane a 2 x 2 block of outputs over a
// quarter of r; the quarters added in a fixed order).  fp32 throughout.
// A and B are functions of the token alone (same section: every token gets
// its own compact vectors), so their rows come either from this cycle's
// projection of the gathered embedding rows or from a per-token table
// built once.
//
// Path (same section; and "DFlash 2 讓 Qwen3.8-27B 快了兩倍", item 2 --
// Viterbi): one work-group per request, whose first wave runs the
// recursion.  VITERBI keeps delta_t[j] = max_i delta_{t-1}[i] + S_t[i][j]
// with back-pointers in LDS: lane l owns target rank j = l >> 2 and four
// predecessors i = 4 (l & 3) + e, and the four lanes of a quad are combined
// with DPP quad permutations (value, lowest rank).
// GREEDY follows the best successor; SAMPLE draws c_t from
// softmax_j(S_t(c_{t-1}, j) / tau) by inverse CDF in rank order with a
// Philox uniform.  Path sums are float additions.
#include "df2_internal.h"
#include "select_body.h"

namespace df2 {
namespace {
using namespace selectd;

// Kernel arguments are ordered so that what a work-group needs first falls
// in the 56 bytes the command processor preloads into SGPRs (no scalar load
// before the first memory request).
__global__ __launch_bounds__(64) void slice_reduce_kernel(float* __restrict__ p0, float* __restrict__ p1,
                                                           float* __restrict__ p2, int n0, int n1, int n2,
                                                           int split, int64_t k0, int64_t k1, int64_t k2) {
  slice_reduce_elem(p0, n0, k0, p1, n1, k1, p2, n2, k2, split, (int64_t)blockIdx.x * 64 + threadIdx.x);
}

template <bool TAB>
__global__ __launch_bounds__(256) void pair_epilogue_kernel(const float* __restrict__ ab,
                                                            const float* __restrict__ a_last,
                                                            const float* __restrict__ h_part,
                                                            const float* __restrict__ cand_val, int T, int K,
                                                            int r, int gate, float* __restrict__ scores,
                                                            const int32_t* __restrict__ cand_idx,
                                                            const int32_t* __restrict__ last_tok, int64_t vocab,
                                                            int hsplit, int64_t h_k) {
  __shared__ PairLds<TAB> L;
  pair_epilogue_body<TAB>(ab, a_last, h_part, gate, cand_val, cand_idx, last_tok, vocab, hsplit, h_k, T, K, r,
                          scores, blockIdx.x, L);
}

__global__ __launch_bounds__(kPathThreads) void path_kernel(const float* __restrict__ scores,
                                                            const int32_t* __restrict__ cand_idx, int T, int K,
                                                            int mode, float inv_tau,
                                                            const uint64_t* __restrict__ seed_dev, int b0,
                                                            int32_t* __restrict__ path_rank,
                                                            int32_t* __restrict__ path_tok, float* __restrict__ q,
                                                            float* __restrict__ path_score) {
  __shared__ PathLds L;
  path_body(scores, cand_idx, T, K, mode, inv_tau, seed_dev, b0, path_rank, path_tok, q, path_score, blockIdx.x,
            L);
}

}  // namespace

hipError_t launch_pair_epilogue(float* ab, float* a_last, float* h, int split,
                                int64_t ab_k, int64_t alast_k, int64_t h_k, int gate,
                                const float* cand_val, int B, int T, int K, int r, float* scores,
                                hipStream_t stream) {
  if (B * T == 0) return hipSuccess;
  if (split > 1) {
    // sum the slices into slice 0 over many work-groups first; the epilogue
    // then reads one slice
    const int64_t n0 = (int64_t)B * T * K * 2 * r / 4, n1 = (int64_t)B * r / 4, n2 = (int64_t)B * T * r / 4;
    const int64_t n = n0 + n1 + n2;
    // a split projection has few tiles, so n is far below 2^31 (the kernel
    // takes the counts as int)
    if (n >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    ProfileScope pr("proj_reduce", stream);
    DF2_TRY(launch(slice_reduce_kernel, dim3((unsigned)((n + 63) / 64)), dim3(64), 0, stream, pr,
                   ab, a_last, h, (int)n0, (int)n1, (int)n2, split, ab_k, alast_k, h_k));
  }
  ProfileScope ps("pair_epilogue", stream);
  DF2_TRY(launch(pair_epilogue_kernel<false>, dim3(B * T), dim3(256), 0, stream, ps, ab, a_last, h, cand_val, T, K,
                 r, gate, scores, (const int32_t*)nullptr, (const int32_t*)nullptr, (int64_t)0, 1, (int64_t)0));
  return hipGetLastError();
}

hipError_t launch_pair_epilogue_tab(const float* tab, int64_t vocab, const int32_t* cand_idx,
                                    const int32_t* last_tok, const float* h, int split, int64_t h_k, int gate,
                                    const float* cand_val, int B, int T, int K, int r, float* scores,
                                    hipStream_t stream) {
  if (B * T == 0) return hipSuccess;
  ProfileScope ps("pair_epilogue", stream);
  DF2_TRY(launch(pair_epilogue_kernel<true>, dim3(B * T), dim3(256), 0, stream, ps, tab, (const float*)nullptr,
                 h, cand_val, T, K, r, gate, scores, cand_idx, last_tok, vocab, split, h_k));
  return hipGetLastError();
}

hipError_t launch_path(const float* scores, const int32_t* cand_idx, int B, int T, int K, int mode,
                       float temperature, const uint64_t* seed_dev, int b0, int32_t* path_rank,
                       int32_t* path_tok, float* q, float* path_score, hipStream_t stream) {
  if (B == 0) return hipSuccess;
  float inv_tau = mode == 2 ? 1.0f / temperature : 0.f;
  ProfileScope ps("path", stream);
  DF2_TRY(launch(path_kernel, dim3(B), dim3(kPathThreads), 0, stream, ps, scores, cand_idx, T, K, mode, inv_tau, seed_dev,
                                                b0, path_rank, path_tok, q, path_score));
  return hipGetLastError();
}

}  // namespace df2

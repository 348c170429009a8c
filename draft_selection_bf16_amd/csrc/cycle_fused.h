// cycle_fused.h -- arguments of the persistent small-batch cycle kernel
// (cycle_fused.hip).  Internal; not part of the ABI.
#pragma once

#include "gemm_tile.h"

namespace df2 {

struct FusedArgs {
  // drafter block logits [B T, vocab] and target logits [B (T+1), vocab], bf16
  const void* logits;
  const void* target;
  int64_t vocab;
  int B, T, K, r, gate, mode;   // mode: path VITERBI (0) or GREEDY (1)
  // top-K: chunks per row, chunk length, per-chunk lists; the candidates
  int tsplits;
  int64_t tchunk;
  uint64_t* tpart;
  int32_t* cand_idx;
  float* cand_val;
  // projection: the problem (P.ksplit set by the caller, the rest by the
  // launcher) and the slices of its products, as the pair-score epilogue
  // reads them
  gemm::Problem P;
  float* ab;
  float* alast;
  float* hg;
  int64_t ab_k, alast_k, h_k;   // floats between slices
  int64_t n0, n1, n2;           // float4 per slice of ab, alast, hg
  float* scores;
  int32_t* path_rank;
  int32_t* path_tok;
  float* q;
  float* path_score;            // may be null
  // greedy verification: chunks per target row, chunk length, partials
  int vsplits;
  int64_t vchunk;
  uint64_t* vpart;
  int32_t* accept_len;
  int32_t* out_tok;
  // control words (fused_ctr_bytes) and the launch's status word
  uint32_t* ctr;
  int32_t* status;
  // filled by the launcher
  int rows, free_tiles, nproj, nargmax, nreduce;
  int base_argmax, base_proj, base_reduce, base_pair, base_path, total;
};

// chunking of the fused launch's top-K and argmax passes (their results do
// not depend on it)
TopkPlan fused_topk_plan(int64_t rows, int64_t vocab, int k);
int fused_verify_splits(int B, int T, int64_t vocab, int64_t& chunk);
// bytes of control words for B T rows (zero before the first launch)
size_t fused_ctr_bytes(int rows);
hipError_t launch_fused_ctr_clear(void* ctr, int rows, hipStream_t stream);
// segs: the projection problems in the order [A(last), H, B(cand), A(cand)]
hipError_t launch_cycle_fused(FusedArgs a, const GemmSeg* segs, int d, hipStream_t stream);

}  // namespace df2

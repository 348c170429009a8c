// cycle_fused.hip -- a whole small-batch cycle (top-K, projection, pair
// scores, path, greedy verification) in one persistent launch.
//
// At batch 1 every stage of the cycle is short and latency-bound, and the
// time between dependent launches is a large part of the cycle (the pages
// show decoding speed set by launch overhead: "DFlash 2 讓 Qwen3.8-27B 快了兩倍",
// 坑 6, with and without the decode graph).  Here the stages run as work-groups
// of one launch and wait for each other through counters instead of kernel
// boundaries.  The arithmetic is that of the stage kernels (the same device
// bodies, the same K split and summation orders), so the results equal
// the multi-launch cycle's bit for bit.
//
// Measured at batch 1 / block 8 (V = 151,936, d = 5120): 61.2-61.3 us per
// replayed cycle against 41.7 us for the eight-kernel graph (63.6-65.2
// against 46.0 us with the streaming top-K body in both).  A dependent
// launch inside a replayed graph costs only about 1-2 us on this part, while
// each stage body has 5-15 us of latency of its own (3.5-6 us for a launch
// whose work-groups do nothing), and every wait on another work-group (its
// release, the counter round trip, the poll, the acquire) costs about what
// the launch gap it replaces did.  The multi-launch graph stays the default.
//
// Scheduling.  Every work-group draws a ticket from a counter when it starts
// and the ticket picks its work: tickets [0, nA) scan top-K chunks, then
// come projection tiles, slice sums, pair-score rows, the target's argmax
// chunks and finally one path + verification work-group per request.  A work-group
// waits only for work of lower tickets, which started before it and waits
// only for lower tickets again, so every wait ends whatever the number of
// work-groups resident at a time.  Waits poll a counter with relaxed
// agent-scope loads and a bounded spin (a time-out sets an error word that
// the launch reports in `status`); a producer makes its writes visible at
// agent scope (its waves' stores complete, then one L2 write-back) before it
// counts itself, a consumer acquires (one invalidation) after its wait.  The last chunk of a row to finish
// merges the row's lists (no wait at all); the work-group that finishes
// last resets every counter for the next launch.
#include "cycle_fused.h"
#include "select_body.h"
#include "topk_body.h"
#include "verify_body.h"

namespace df2 {
namespace {

constexpr int kNW = 4;                   // waves per work-group
constexpr int kThreads = kNW * kWave;
constexpr int kTopkEpt = 20;             // entries per thread of the short-chunk top-K
constexpr int kPBM = 64, kPBN = 128, kPS = 3;   // projection tiles (64 x 128, 3 LDS stages)
constexpr int kSpinLimit = 1 << 22;      // polls before a wait gives up
static_assert(verifyd::kThreads == kThreads && selectd::kPathThreads == kThreads, "one work-group size");

// control words, 64 bytes apart
enum : int { C_TICKET = 0, C_MERGED, C_PROJ, C_RED, C_PAIR, C_ARGMAX, C_EXIT, C_ERR, C_ROW };
constexpr int kCtrStride = 16;

__device__ __forceinline__ uint32_t ctr_add(uint32_t* c, uint32_t v) {
  return __hip_atomic_fetch_add(c, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ctr_load(uint32_t* c) {
  return __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Every wave's stores complete (work-group release), then thread 0 makes
// them visible at agent scope (one L2 write-back for the work-group) and
// counts the work-group.
__device__ __forceinline__ void signal(uint32_t* c) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    ctr_add(c, 1u);
  }
}

// thread 0 polls until *c >= target (bounded) -- few, widely spaced reads,
// so that the pollers do not slow the producers' own counter updates --
// then acquires at agent scope for the work-group (its waves read after the
// barrier, through the caches that acquire invalidated)
__device__ __forceinline__ bool poll(uint32_t* c, uint32_t target, uint32_t* err) {
  int spins = 0;
  while (ctr_load(c) < target) {
    if (++spins > kSpinLimit) {
      __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
    __builtin_amdgcn_s_sleep(8);
  }
  return true;
}
__device__ __forceinline__ void wait_for(uint32_t* c, uint32_t target, uint32_t* err) {
  if (threadIdx.x == 0) {
    poll(c, target, err);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
}

// the tile a projection work-group runs (the numbering of gemm::run_tile)
__device__ __forceinline__ int proj_tile(int bid, int nb, int ksplit) {
  if (ksplit != 1) return bid / ksplit;
  const int full = nb / 8 * 8;
  return bid < full ? (bid % 8) * (full / 8) + bid / 8 : bid;
}

__global__ __launch_bounds__(kThreads) void cycle_fused_kernel(FusedArgs a) {
  __shared__ int s_vid, s_last;
  uint32_t* ctr = a.ctr;
  uint32_t* err = ctr + C_ERR * kCtrStride;
  if (threadIdx.x == 0) s_vid = (int)ctr_add(ctr + C_TICKET * kCtrStride, 1u);
  __syncthreads();
  const int vid = s_vid;   // the same in the whole work-group
  if (vid >= a.total) {     // control words not zero at the launch: no work, report
    if (threadIdx.x == 0) __hip_atomic_store(a.status, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }

  if (vid < a.base_proj) {
    // ---- top-K of one chunk of one drafter row; the row's last chunk merges
    if (a.tchunk <= (int64_t)kThreads * kTopkEpt) {   // one round of loads per chunk
      auto& L = *reinterpret_cast<topkd::TopkSmallLds<kNW>*>(dyn_lds);
      topkd::topk_small_body<topkd::Bf16, kNW, kTopkEpt>(a.logits, a.vocab, a.tsplits, a.tchunk, a.K, a.cand_idx,
                                                         a.cand_val, a.tpart, vid, L);
    } else {
      auto& L = *reinterpret_cast<topkd::TopkChunkLds<kNW>*>(dyn_lds);
      topkd::topk_chunk_body<topkd::Bf16, kNW>(a.logits, a.vocab, a.tsplits, a.tchunk, a.K, a.cand_idx, a.cand_val,
                                               a.tpart, vid, L);
    }
    if (a.tsplits == 1) {
      signal(ctr + C_MERGED * kCtrStride);
    } else {
      const int row = vid / a.tsplits;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __syncthreads();
      if (threadIdx.x == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        s_last = ctr_add(ctr + (C_ROW + row) * kCtrStride, 1u) == (uint32_t)(a.tsplits - 1) ? 1 : 0;
        if (s_last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      }
      __syncthreads();
      if (s_last) {
        if (wave_id() == 0) {
          uint64_t* sel = (uint64_t*)dyn_lds;
          topkd::topk_merge_row(a.tpart, row, a.tsplits, a.K, a.cand_idx, a.cand_val, sel, sel + 16);
        }
        signal(ctr + C_MERGED * kCtrStride);
      }
    }
  } else if (vid < a.base_reduce) {
    // ---- one projection tile (one K slice); candidate rows wait for the merges
    const int bid = vid - a.base_proj;
    if (proj_tile(bid, a.nproj, a.P.ksplit) >= a.free_tiles) wait_for(ctr + C_MERGED * kCtrStride, a.rows, err);
    gemm::run_tile<kPBM, kPBN, kPS, kNW, 1, false>(a.P, bid, a.nproj);   // read in this launch: cached stores
    signal(ctr + C_PROJ * kCtrStride);
  } else if (vid < a.base_pair) {
    // ---- slices summed into slice 0, one float4 per thread
    wait_for(ctr + C_PROJ * kCtrStride, a.nproj, err);
    const int64_t e = (int64_t)(vid - a.base_reduce) * kThreads + threadIdx.x;
    selectd::slice_reduce_elem(a.ab, a.n0, a.ab_k, a.alast, a.n1, a.alast_k, a.hg, a.n2, a.h_k, a.P.ksplit, e);
    signal(ctr + C_RED * kCtrStride);
  } else if (vid < a.base_argmax) {
    // ---- pair scores of one (request, position)
    if (a.nreduce > 0)
      wait_for(ctr + C_RED * kCtrStride, a.nreduce, err);
    else
      wait_for(ctr + C_PROJ * kCtrStride, a.nproj, err);
    auto& L = *reinterpret_cast<selectd::PairLds<false>*>(dyn_lds);
    selectd::pair_epilogue_body<false>(a.ab, a.alast, a.hg, a.gate, a.cand_val, nullptr, nullptr, 0, 1, 0, a.T, a.K,
                                       a.r, a.scores, vid - a.base_pair, L);
    signal(ctr + C_PAIR * kCtrStride);
  } else if (vid < a.base_path) {
    // ---- argmax partial of one chunk of one target row
    verifyd::argmax_part_body<1>(a.target, a.vocab, a.vsplits, a.vchunk, a.vpart, vid - a.base_argmax,
                                 (uint64_t*)dyn_lds);
    signal(ctr + C_ARGMAX * kCtrStride);
  } else {
    // ---- path of one request, then its greedy verification (first wave)
    const int b = vid - a.base_path;
    wait_for(ctr + C_PAIR * kCtrStride, a.rows, err);
    auto& L = *reinterpret_cast<selectd::PathLds*>(dyn_lds);
    selectd::path_body(a.scores, a.cand_idx, a.T, a.K, a.mode, 0.f, nullptr, 0, a.path_rank, a.path_tok, a.q,
                       a.path_score, b, L);
    if (wave_id() == 0) {
      if (lane_id() == 0) poll(ctr + C_ARGMAX * kCtrStride, (uint32_t)a.nargmax, err);
      // the path just written by this wave and the other work-groups'
      // argmax partials
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "agent");
      verifyd::greedy_final_body(a.vpart, a.vsplits, a.T, a.path_tok, a.accept_len, a.out_tok, b);
    }
  }

  // ---- the last work-group to finish reports and resets the counters
  __syncthreads();
  if (threadIdx.x == 0 && ctr_add(ctr + C_EXIT * kCtrStride, 1u) == (uint32_t)(a.total - 1)) {
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    a.status[0] = (int32_t)ctr_load(err);
    for (int c = 0; c < C_ROW + a.rows; ++c)
      __hip_atomic_store(ctr + c * kCtrStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// zero the control words (before the first launch on a workspace)
__global__ __launch_bounds__(256) void fused_ctr_clear_kernel(uint32_t* ctr, int n) {
  for (int i = threadIdx.x; i < n; i += 256) ctr[i] = 0u;
}

bool g_lds_set = false;

constexpr size_t lds_bytes() {
  size_t m = (size_t)kPS * (kPBM + kPBN) * mfma::BK * 2;
  m = sizeof(topkd::TopkChunkLds<kNW>) > m ? sizeof(topkd::TopkChunkLds<kNW>) : m;
  m = sizeof(topkd::TopkSmallLds<kNW>) > m ? sizeof(topkd::TopkSmallLds<kNW>) : m;
  m = sizeof(selectd::PairLds<false>) > m ? sizeof(selectd::PairLds<false>) : m;
  m = sizeof(selectd::PathLds) > m ? sizeof(selectd::PathLds) : m;
  return m;
}

}  // namespace

// Top-K: the stand-alone plan's chunks halved (four waves scan a chunk
// here, eight there), at most 32 per row (the merge's limit).
TopkPlan fused_topk_plan(int64_t rows, int64_t vocab, int k) {
  TopkPlan p = topk_plan(rows, vocab, k);
  if (p.splits > 1) {
    int64_t s = 2 * (int64_t)p.splits;
    if (s > 32) s = 32;
    int64_t chunk = (vocab + s - 1) / s;
    chunk = (chunk + 63) / 64 * 64;
    p.splits = (int)((vocab + chunk - 1) / chunk);
    p.chunk = chunk;
    p.ws_bytes = align256((size_t)rows * (size_t)p.splits * 16 * sizeof(uint64_t));
  }
  p.small = 0;   // (the persistent launch picks its chunk body by the chunk's length)
  return p;
}

// Argmax of the target rows: off the critical path (only the last step
// reads it), so long chunks of >= kArgChunk entries and few work-groups.
constexpr int64_t kArgChunk = 32768;
int fused_verify_splits(int B, int T, int64_t vocab, int64_t& chunk) {
  (void)B;
  (void)T;
  int64_t s = (vocab + kArgChunk - 1) / kArgChunk;
  if (s < 1) s = 1;
  chunk = (vocab + s - 1) / s;
  chunk = (chunk + 63) / 64 * 64;
  return (int)((vocab + chunk - 1) / chunk);
}

size_t fused_ctr_bytes(int rows) { return (size_t)(C_ROW + rows) * kCtrStride * sizeof(uint32_t); }

hipError_t launch_fused_ctr_clear(void* ctr, int rows, hipStream_t stream) {
  ProfileScope ps("fused_clear", stream);
  DF2_TRY(launch(fused_ctr_clear_kernel, dim3(1), dim3(256), 0, stream, ps, (uint32_t*)ctr,
                 (C_ROW + rows) * kCtrStride));
  return hipGetLastError();
}

// Fill the stage bases and the projection problem of `a` (the caller set
// the pointers, shapes and plans) and launch.
hipError_t launch_cycle_fused(FusedArgs a, const GemmSeg* segs, int d, hipStream_t stream) {
  if (a.B == 0) return hipSuccess;
  int tiles = 0;
  DF2_TRY(gemm::make_problem(segs, 4, d, a.P.ksplit, kPBM, kPBN, a.P, tiles));
  // segments 0 and 1 (the last tokens' A and H) need no candidates
  a.free_tiles = a.P.tile_begin[2];
  a.rows = a.B * a.T;
  a.nproj = tiles * a.P.ksplit;
  a.nargmax = a.B * (a.T + 1) * a.vsplits;
  const int64_t n4 = a.n0 + a.n1 + a.n2;
  a.nreduce = a.P.ksplit > 1 ? (int)((n4 + kThreads - 1) / kThreads) : 0;
  // the chain top-K -> projection -> slice sums -> pair scores first; the
  // target's argmax chunks (needed only by the last step) fill in after it
  a.base_proj = a.rows * a.tsplits;
  a.base_reduce = a.base_proj + a.nproj;
  a.base_pair = a.base_reduce + a.nreduce;
  a.base_argmax = a.base_pair + a.rows;
  a.base_path = a.base_argmax + a.nargmax;
  a.total = a.base_path + a.B;
  constexpr size_t kLds = lds_bytes();
  static_assert(kLds + 64 <= 160 * 1024, "LDS of one work-group");
  if (!g_lds_set) {
    hipError_t e = hipFuncSetAttribute((const void*)cycle_fused_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)kLds);
    if (e != hipSuccess) return e;
    g_lds_set = true;
  }
  ProfileScope ps("cycle_fused", stream);
  DF2_TRY(launch(cycle_fused_kernel, dim3((unsigned)a.total), dim3(kThreads), (unsigned)kLds, stream, ps, a));
  return hipGetLastError();
}

}  // namespace df2

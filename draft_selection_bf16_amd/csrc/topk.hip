// topk.hip -- K best entries of every row of a logits matrix (K <= 16).
//
// DFlash 2 keeps the 16 best candidates of each draft position ("DFlash 2:
// Keep Drafting Parallel", sections "The right tokens are already there" and
// "A lightweight path selector").  Order: value descending, equal values by
// lower index.
//
// Design (HBM-streaming, one pass over the logits):
//  * each row is cut into `splits` contiguous chunks (one per row once there
//    are a few hundred rows); one 512-thread work-group per (row, chunk);
//    its eight waves stream interleaved 1 KB slices with 16-byte loads
//    (8 bf16 / 4 fp32 per lane), four loads in flight per lane;
//  * every wave filters against a threshold: the largest value any wave of
//    the work-group has published as a lower bound of its own 16th best (any
//    such bound is a bound for the work-group).  For bf16 rows and a
//    positive threshold the check is a packed signed 16-bit maximum of the
//    eight raw values against the threshold's bits (order-preserving there),
//    about seven instructions per 16-byte load;
//  * a 16-byte group that may hold a candidate is queued raw in a per-wave
//    LDS queue (a few instructions); a full queue is expanded in bulk, one
//    group per lane, into exact 64-bit (value, index) keys in a per-wave LDS
//    buffer, which is then cut back with a search over the value bits only
//    (ballot popcounts on the scalar unit; ties kept) -- this raises the
//    threshold to the 16th best value seen so far;
//  * at the end each wave ranks its remaining keys (a few dozen) and keeps
//    its 16 best, and one wave ranks those 8 x 16 (each key's rank is the
//    number of larger keys: independent compares, no serial search); with
//    one chunk per row it writes the result in order, otherwise a second
//    kernel merges the per-chunk lists of each row.
// (value, index) pairs are compared as single 64-bit keys (df2_device.h), so
// the result does not depend on the order in which entries are seen.
#include "df2_internal.h"
#include "topk_body.h"

namespace df2 {
namespace {
using namespace topkd;

constexpr int kWaves = 8;        // waves per work-group
constexpr int kThreads = kWaves * kWave;
constexpr int kSmallEpt = 16;    // entries per thread of the short-chunk path
constexpr int64_t kSmallChunk = (int64_t)kThreads * kSmallEpt;

template <typename E>
__global__ __launch_bounds__(kThreads) void topk_chunk_kernel(
    const void* __restrict__ logits, int64_t vocab, int splits, int64_t chunk, int k,
    int32_t* __restrict__ out_idx, float* __restrict__ out_val, uint64_t* __restrict__ part) {
  __shared__ TopkChunkLds<kWaves> L;
  topk_chunk_body<E, kWaves>(logits, vocab, splits, chunk, k, out_idx, out_val, part, blockIdx.x, L);
}

template <typename E>
__global__ __launch_bounds__(kThreads) void topk_small_kernel(
    const void* __restrict__ logits, int64_t vocab, int splits, int64_t chunk, int k,
    int32_t* __restrict__ out_idx, float* __restrict__ out_val, uint64_t* __restrict__ part) {
  __shared__ TopkSmallLds<kWaves> L;
  topk_small_body<E, kWaves, kSmallEpt>(logits, vocab, splits, chunk, k, out_idx, out_val, part, blockIdx.x, L);
}

// one row per work-group of one wave (grid = rows)
__global__ __launch_bounds__(kWave) void topk_merge_kernel(const uint64_t* __restrict__ part, int splits, int k,
                                                           int32_t* __restrict__ out_idx,
                                                           float* __restrict__ out_val) {
  __shared__ uint64_t sel[16];
  __shared__ __attribute__((aligned(16))) uint64_t ssv[kWave];
  topk_merge_row(part, (int64_t)blockIdx.x, splits, k, out_idx, out_val, sel, ssv);
}

}  // namespace

TopkPlan topk_plan(int64_t rows, int64_t vocab, int k) {
  (void)k;
  // One work-group of eight waves per row and no merge from 256 rows on (at
  // 480 rows most CUs scan two rows).  Below that, as many chunks per row as
  // keep rows * chunks <= 256, one work-group per CU: a CU's share of the
  // bytes is what bounds the scan, and every chunk adds a fixed cost
  // (priming, the final selection) and 16 keys to merge.  Measured per
  // cycle against the earlier target of ~448 work-groups: 224 rows 98.5
  // against 101.2 us (1 chunk instead of 2), 120 rows 79.7 against 81.3
  // (2 instead of 4), 56 rows 100.3 against 101.1 (4 instead of 8), 15 rows
  // 55.8 against 58.6 (17 instead of 18).  Chunks stay >= 8192 entries and
  // <= 32 per row (the merge holds at most 512 keys per row).
  // With few rows, chunks of at most kSmallChunk entries on the short-chunk
  // path instead (one round of loads per work-group), up to about four
  // work-groups per CU.  Per cycle against the long path: 7 rows (133
  // work-groups) 41.5 against 45.6 us, 15 rows 49.6 against 52.4, 56 rows
  // (1,064) 89.5 against 93.0; 120 rows (2,280) 80.6 against 76.5 and 224
  // rows (4,256) 107 against 89.5 stay on the long path.
  constexpr int64_t kCUs = 256;   // MI355X
  constexpr int64_t kSmallMaxGroups = 1100;
  const int64_t s_small = (vocab + kSmallChunk - 1) / kSmallChunk;
  if (s_small <= 32 && rows * s_small <= kSmallMaxGroups) {
    int64_t chunk = (vocab + s_small - 1) / s_small;
    chunk = (chunk + 63) / 64 * 64;   // <= kSmallChunk (a multiple of 64)
    TopkPlan p;
    p.splits = (int)((vocab + chunk - 1) / chunk);
    p.chunk = chunk;
    p.small = 1;
    p.ws_bytes = p.splits > 1 ? align256((size_t)rows * (size_t)p.splits * 16 * sizeof(uint64_t)) : 0;
    return p;
  }
  int64_t want = kCUs / (rows > 0 ? rows : 1);
  int64_t max_by_size = vocab / 8192;
  int64_t s = want < max_by_size ? want : max_by_size;
  if (s < 1) s = 1;
  if (s > 32) s = 32;
  int64_t chunk = (vocab + s - 1) / s;
  chunk = (chunk + 63) / 64 * 64;
  s = (vocab + chunk - 1) / chunk;
  TopkPlan p;
  p.splits = (int)s;
  p.chunk = chunk;
  p.small = 0;
  p.ws_bytes = s > 1 ? align256((size_t)rows * (size_t)s * 16 * sizeof(uint64_t)) : 0;
  return p;
}

hipError_t launch_topk(const void* logits, int dt, int64_t rows, int64_t vocab, int k,
                       int32_t* out_idx, float* out_val, void* ws, const TopkPlan& plan,
                       hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  uint64_t* part = (uint64_t*)ws;
  dim3 grid((unsigned)(rows * plan.splits)), block(kThreads);
  if (plan.small) {
    ProfileScope ps("topk_chunk", stream);
    if (dt == 0)
      DF2_TRY(launch(topk_small_kernel<float>, grid, block, 0, stream, ps, logits, vocab, plan.splits, plan.chunk, k,
                                                           out_idx, out_val, part));
    else if (dt == 1)
      DF2_TRY(launch(topk_small_kernel<Bf16>, grid, block, 0, stream, ps, logits, vocab, plan.splits, plan.chunk, k,
                                                          out_idx, out_val, part));
    else
      DF2_TRY(launch(topk_small_kernel<F16>, grid, block, 0, stream, ps, logits, vocab, plan.splits, plan.chunk, k,
                                                         out_idx, out_val, part));
  } else {
    ProfileScope ps("topk_chunk", stream);
    if (dt == 0)
      DF2_TRY(launch(topk_chunk_kernel<float>, grid, block, 0, stream, ps, logits, vocab, plan.splits, plan.chunk, k,
                                                           out_idx, out_val, part));
    else if (dt == 1)
      DF2_TRY(launch(topk_chunk_kernel<Bf16>, grid, block, 0, stream, ps, logits, vocab, plan.splits, plan.chunk, k,
                                                          out_idx, out_val, part));
    else
      DF2_TRY(launch(topk_chunk_kernel<F16>, grid, block, 0, stream, ps, logits, vocab, plan.splits, plan.chunk, k,
                                                         out_idx, out_val, part));
  }
  if (plan.splits > 1) {
    // one wave per row, each in a work-group of its own (rows on as many
    // CUs: batch 1 / block 8 41.35 -> 40.8 us per cycle against eight rows
    // per work-group)
    ProfileScope ps("topk_merge", stream);
    DF2_TRY(launch(topk_merge_kernel, dim3((unsigned)rows), dim3(kWave), 0, stream, ps, part, plan.splits, k, out_idx,
                   out_val));
  }
  return hipGetLastError();
}

}  // namespace df2

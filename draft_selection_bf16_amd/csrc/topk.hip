// topk.hip -- K best entries of every row of a logits matrix (K <= 16).
//
// DFlash 2 keeps the 16 best candidates of each draft position ("DFlash 2:
// Keep Drafting Parallel", sections "The right tokens are already there" and
// "A lightweight path selector").  Order: value descending, equal values by
// lower index.
//
// Design (HBM-streaming, one pass over the logits):
//  * each row is cut into `splits` contiguous chunks; one 256-thread
//    work-group per (row, chunk); its four waves stream interleaved 1 KB
//    slices with 16-byte loads (8 bf16 / 4 fp32 per lane), four loads in
//    flight per lane;
//  * every wave keeps a running threshold -- the largest 16th-best value any
//    wave of the work-group has published -- and checks one maximum per
//    16-byte load against it; only entries at or above it are appended, as
//    exact (value, index) keys, to a per-wave LDS buffer, and a full buffer
//    is cut back to its 16 best keys with wave-wide max reductions;
//  * the four wave lists are merged in LDS; with one chunk per row the
//    result is written directly, otherwise a second small kernel merges the
//    per-chunk lists of each row.
// (value, index) pairs are compared as single 64-bit keys (df2_device.h), so
// the result does not depend on the order in which entries are seen.
#include "df2_device.h"
#include "df2_internal.h"

namespace df2 {
namespace {

constexpr int kWaves = 4;        // waves per work-group
constexpr int kThreads = kWaves * kWave;
constexpr int kCap = 128;        // LDS keys per wave
constexpr int kUnroll = 4;       // 16-byte loads in flight per lane

template <typename E>
struct Vec;
template <>
struct Vec<float> {               // fp32: 4 per 16 bytes
  static constexpr int n = 4;
  __device__ static float get(const u32x4& v, int e) {
    return __uint_as_float(v[e]);
  }
  __device__ static float scalar(const void* p, int64_t i) { return ((const float*)p)[i]; }
};
struct Bf16 {};
template <>
struct Vec<Bf16> {                // bf16: 8 per 16 bytes
  static constexpr int n = 8;
  __device__ static float get(const u32x4& v, int e) {
    uint32_t w = v[e >> 1];
    return (e & 1) ? bf16_hi(w) : bf16_lo(w);
  }
  __device__ static float scalar(const void* p, int64_t i) {
    return bf16_to_f32(((const uint16_t*)p)[i]);
  }
};
struct F16 {};
template <>
struct Vec<F16> {                 // fp16: 8 per 16 bytes
  static constexpr int n = 8;
  __device__ static float get(const u32x4& v, int e) {
    uint32_t w = v[e >> 1];
    return half_to_f32((uint16_t)((e & 1) ? (w >> 16) : (w & 0xffffu)));
  }
  __device__ static float scalar(const void* p, int64_t i) {
    return half_to_f32(((const uint16_t*)p)[i]);
  }
};

// Per-wave filter state.  `buf` is this wave's LDS key buffer; `share` holds
// one published threshold per wave of the work-group.  Any wave's 16th best
// value is a lower bound for the work-group's 16th best, so every wave may
// filter with the largest published value.
struct Filter {
  uint64_t* buf;
  volatile float* share;
  int cnt;
  float thr;   // entries with value < thr cannot be in the result
};

// Cut the buffer back to its 16 best keys; publish and raise the threshold.
__device__ __forceinline__ void compact(Filter& F, int wave) {
  constexpr int PER = kCap / kWave;
  uint64_t keys[PER];
  const int lane = lane_id();
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    int s = lane + i * kWave;
    keys[i] = s < F.cnt ? F.buf[s] : 0ull;
  }
  __builtin_amdgcn_wave_barrier();
  const uint64_t t = kth16<PER>(keys);
  F.cnt = gather_at_least<PER>(keys, t, F.buf);
  if (t != 0ull) {
    const float v = key_value(t);
    if (v > F.thr) F.thr = v;
    if (lane == 0) F.share[wave] = F.thr;
  }
  __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ void refresh(Filter& F) {
#pragma unroll
  for (int w = 0; w < kWaves; ++w) F.thr = fmaxf(F.thr, F.share[w]);
}

// Append the entries of this lane that reach the threshold (one per call);
// wave-uniform control flow, keys built only when some lane passes.
__device__ __forceinline__ void offer(Filter& F, bool valid, float f, uint32_t idx, int wave) {
  bool pass = valid && f >= F.thr;
  uint64_t m = ballot(pass);
  if (m == 0ull) return;
  if (F.cnt + __popcll(m) > kCap) {
    compact(F, wave);
    pass = valid && f >= F.thr;
    m = ballot(pass);
    if (m == 0ull) return;
  }
  if (pass) F.buf[F.cnt + lanes_below(m)] = make_key(f, idx);
  F.cnt += __popcll(m);
  __builtin_amdgcn_wave_barrier();
}

template <typename E>
__device__ __forceinline__ void scan_range(Filter& F, const void* rowp, int64_t lo, int64_t hi,
                                           int wave) {
  constexpr int VN = Vec<E>::n;
  const int lane = lane_id();
  const uintptr_t base = (uintptr_t)rowp;
  const int esz = sizeof(u32x4) / VN;
  // head / tail elements outside 16-byte alignment: wave 0, one per lane
  int64_t a0 = lo, a1 = hi;
  {
    uintptr_t p0 = base + (uintptr_t)lo * esz;
    int64_t head = (int64_t)(((16 - (p0 & 15)) & 15) / esz);
    a0 = lo + head < hi ? lo + head : hi;
    int64_t body = (hi - a0) / VN * VN;
    a1 = a0 + body;
  }
  if (wave == 0) {
    for (int64_t s = lo; s < a0; s += kWave) {
      int64_t i = s + lane;
      bool v = i < a0;
      offer(F, v, v ? Vec<E>::scalar(rowp, i) : 0.f, (uint32_t)i, wave);
    }
    for (int64_t s = a1; s < hi; s += kWave) {
      int64_t i = s + lane;
      bool v = i < hi;
      offer(F, v, v ? Vec<E>::scalar(rowp, i) : 0.f, (uint32_t)i, wave);
    }
  }
  const u32x4* vp = (const u32x4*)(base + (uintptr_t)a0 * esz);
  const int64_t ngroups = (a1 - a0) / VN;   // 16-byte groups
  const int64_t stride = (int64_t)kWaves * kWave;
  for (int64_t g0 = (int64_t)wave * kWave; g0 < ngroups; g0 += stride * kUnroll) {
    u32x4 v[kUnroll];
    bool ok[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      int64_t g = g0 + u * stride + lane;
      ok[u] = g < ngroups;
      v[u] = ok[u] ? __builtin_nontemporal_load(vp + g) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      float f[VN];
#pragma unroll
      for (int e = 0; e < VN; ++e) f[e] = Vec<E>::get(v[u], e);
      float gm = f[0];
#pragma unroll
      for (int e = 1; e < VN; ++e) gm = fmaxf(gm, f[e]);
      if (ballot(ok[u] && gm >= F.thr) == 0ull) continue;
      const uint32_t i0 = (uint32_t)(a0 + (g0 + u * stride + lane) * VN);
#pragma unroll
      for (int e = 0; e < VN; ++e) offer(F, ok[u], f[e], i0 + e, wave);
    }
    refresh(F);
  }
}

// grid: rows * splits work-groups of kThreads.  If splits == 1 writes the
// final k results, else the 16 best keys of the chunk to part.
template <typename E>
__global__ __launch_bounds__(kThreads) void topk_chunk_kernel(
    const void* __restrict__ logits, int64_t vocab, int splits, int64_t chunk, int k,
    int32_t* __restrict__ out_idx, float* __restrict__ out_val, uint64_t* __restrict__ part) {
  __shared__ uint64_t sbuf[kWaves][kCap];
  __shared__ uint64_t smerge[kWaves * 16];
  __shared__ float sthr[kWaves];
  const int wave = threadIdx.x / kWave, lane = lane_id();
  const int64_t row = blockIdx.x / splits;
  const int split = blockIdx.x % splits;
  const int64_t lo = (int64_t)split * chunk;
  const int64_t hi = lo + chunk < vocab ? lo + chunk : vocab;
  const int esz = sizeof(u32x4) / Vec<E>::n;
  const void* rowp = (const char*)logits + row * vocab * esz;

  if (lane == 0) sthr[wave] = -INFINITY;
  __syncthreads();
  Filter F{sbuf[wave], sthr, 0, -INFINITY};
  scan_range<E>(F, rowp, lo, hi, wave);
  compact(F, wave);
  if (lane < 16) smerge[wave * 16 + lane] = lane < F.cnt ? F.buf[lane] : 0ull;
  __syncthreads();
  if (wave != 0) return;
  uint64_t keys[1] = {smerge[lane]};
  const uint64_t t = kth16<1>(keys);
  __builtin_amdgcn_wave_barrier();
  const int n = gather_at_least<1>(keys, t, smerge);
  __builtin_amdgcn_wave_barrier();
  if (splits == 1) {
    const uint64_t mine = sorted16(smerge, n);
    if (lane < k) {
      out_idx[row * k + lane] = (int32_t)key_index(mine);
      out_val[row * k + lane] = key_value(mine);
    }
  } else if (lane < 16) {
    part[((int64_t)row * splits + split) * 16 + lane] = lane < n ? smerge[lane] : 0ull;
  }
}

// one wave per row: merge splits * 16 keys (splits <= 32)
__global__ __launch_bounds__(kThreads) void topk_merge_kernel(const uint64_t* __restrict__ part,
                                                              int64_t rows, int splits, int k,
                                                              int32_t* __restrict__ out_idx,
                                                              float* __restrict__ out_val) {
  constexpr int PER = 8;
  __shared__ uint64_t sel[kWaves][16];
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int64_t row = (int64_t)blockIdx.x * kWaves + wave;
  if (row >= rows) return;
  const int n = splits * 16;
  uint64_t keys[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    int s = lane + i * kWave;
    keys[i] = s < n ? part[row * n + s] : 0ull;
  }
  const uint64_t t = kth16<PER>(keys);
  const int m = gather_at_least<PER>(keys, t, sel[wave]);
  __builtin_amdgcn_wave_barrier();
  const uint64_t mine = sorted16(sel[wave], m);
  if (lane < k) {
    out_idx[row * k + lane] = (int32_t)key_index(mine);
    out_val[row * k + lane] = key_value(mine);
  }
}

}  // namespace

TopkPlan topk_plan(int64_t rows, int64_t vocab, int k) {
  (void)k;
  // aim for >= 2048 work-groups, but keep chunks >= 16K entries and
  // <= 32 chunks per row (the merge holds at most 512 keys per row)
  int64_t want = (2048 + rows - 1) / (rows > 0 ? rows : 1);
  int64_t max_by_size = vocab / 16384;
  int64_t s = want < max_by_size ? want : max_by_size;
  if (s < 1) s = 1;
  if (s > 32) s = 32;
  int64_t chunk = (vocab + s - 1) / s;
  chunk = (chunk + 63) / 64 * 64;
  s = (vocab + chunk - 1) / chunk;
  TopkPlan p;
  p.splits = (int)s;
  p.chunk = chunk;
  p.ws_bytes = s > 1 ? align256((size_t)rows * (size_t)s * 16 * sizeof(uint64_t)) : 0;
  return p;
}

hipError_t launch_topk(const void* logits, int dt, int64_t rows, int64_t vocab, int k,
                       int32_t* out_idx, float* out_val, void* ws, const TopkPlan& plan,
                       hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  uint64_t* part = (uint64_t*)ws;
  dim3 grid((unsigned)(rows * plan.splits)), block(kThreads);
  {
    ProfileScope ps("topk_chunk", stream);
    if (dt == 0)
      topk_chunk_kernel<float><<<grid, block, 0, stream>>>(logits, vocab, plan.splits, plan.chunk, k,
                                                           out_idx, out_val, part);
    else if (dt == 1)
      topk_chunk_kernel<Bf16><<<grid, block, 0, stream>>>(logits, vocab, plan.splits, plan.chunk, k,
                                                          out_idx, out_val, part);
    else
      topk_chunk_kernel<F16><<<grid, block, 0, stream>>>(logits, vocab, plan.splits, plan.chunk, k,
                                                         out_idx, out_val, part);
  }
  if (plan.splits > 1) {
    ProfileScope ps("topk_merge", stream);
    dim3 g2((unsigned)((rows + kWaves - 1) / kWaves));
    topk_merge_kernel<<<g2, block, 0, stream>>>(part, rows, plan.splits, k, out_idx, out_val);
  }
  return hipGetLastError();
}

}  // namespace df2

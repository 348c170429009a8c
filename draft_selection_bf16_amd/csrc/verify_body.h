// verify_body.h -- device code shared by the verification kernels
// (verify.hip) and the persistent cycle kernel: element access, the row
// streaming loop, the argmax partial of one (row, chunk) work-group and the
// greedy decision of one request, as device functions that take their block
// index and LDS from the caller.  Internal; not part of the ABI.
#pragma once

#include "df2_device.h"
#include "df2_internal.h"

namespace df2 {
namespace verifyd {


constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kUnroll = 4;
constexpr float kLog2e = 1.4426950408889634f;

struct DecRec {  // per-request decision of the rejection pass
  int n;         // accepted drafts; the row that is (re)sampled
  int argmax;    // lowest argmax of that row (fallback when no mass)
  float m, s;    // row max and sum of exp2((z - m) c)
  float u2;      // the uniform of the draw
  float pad;
};

struct RowPart {  // streaming partial of one chunk of one row
  uint64_t key;   // (max value, lowest index) of the chunk
  float s;        // sum of exp2((z - value(key)) c) over the chunk
  float pad;
};

template <int DT>
struct Elt;
template <>
struct Elt<0> {
  static constexpr int VN = 4, ESZ = 4;
  __device__ static float vget(const u32x4& v, int e) { return __uint_as_float(v[e]); }
  __device__ static float one(const void* p, int64_t i) { return ((const float*)p)[i]; }
};
template <>
struct Elt<1> {
  static constexpr int VN = 8, ESZ = 2;
  __device__ static float vget(const u32x4& v, int e) {
    uint32_t w = v[e >> 1];
    return (e & 1) ? bf16_hi(w) : bf16_lo(w);
  }
  __device__ static float one(const void* p, int64_t i) { return bf16_to_f32(((const uint16_t*)p)[i]); }
};
template <>
struct Elt<2> {
  static constexpr int VN = 8, ESZ = 2;
  __device__ static float vget(const u32x4& v, int e) {
    uint32_t w = v[e >> 1];
    return half_to_f32((uint16_t)((e & 1) ? (w >> 16) : (w & 0xffffu)));
  }
  __device__ static float one(const void* p, int64_t i) { return half_to_f32(((const uint16_t*)p)[i]); }
};

// Visit elements [lo, hi) of a row: scalar head/tail up to 16-byte
// alignment, vector body with kUnroll loads in flight per thread.  Within a
// thread the visiting order is increasing in index.
template <int DT, typename F>
__device__ __forceinline__ void stream_row(const void* rowp, int64_t lo, int64_t hi, F& f) {
  using E = Elt<DT>;
  const int tid = threadIdx.x;
  const unsigned mis = (unsigned)(size_t)((const char*)rowp + lo * E::ESZ) & 15u;
  int64_t head = (int64_t)(((16u - mis) & 15u) / E::ESZ);
  int64_t a0 = lo + head < hi ? lo + head : hi;
  int64_t a1 = a0 + (hi - a0) / E::VN * E::VN;
  for (int64_t i = lo + tid; i < a0; i += kThreads) f.one(E::one(rowp, i), i);
  const u32x4* vp = (const u32x4*)((const char*)rowp + a0 * E::ESZ);
  const int64_t ng = (a1 - a0) / E::VN;
  for (int64_t g0 = tid; g0 < ng; g0 += (int64_t)kThreads * kUnroll) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      // unconditional (clamped) loads keep all kUnroll loads in flight
      int64_t g = g0 + (int64_t)u * kThreads;
      v[u] = __builtin_nontemporal_load(vp + (g < ng ? g : 0));
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      int64_t g = g0 + (int64_t)u * kThreads;
      if (g < ng) f.template vec<DT>(v[u], a0 + g * E::VN);
    }
  }
  for (int64_t i = a1 + tid; i < hi; i += kThreads) f.one(E::one(rowp, i), i);
}

template <int DT, typename F>
__device__ __forceinline__ void vec_as_floats(F& f, const u32x4& v, int64_t i0) {
  using E = Elt<DT>;
  float x[E::VN];
#pragma unroll
  for (int e = 0; e < E::VN; ++e) x[e] = E::vget(v, e);
  f.template group<E::VN>(x, i0);
}

// ---------------------------------------------------------------- argmax
typedef short s16x2 __attribute__((ext_vector_type(2)));

// Largest of the eight bf16 values of v as a signed 16-bit integer: for
// positive values this orders like the value, every negative value (and -0)
// is negative.  (Words are reinterpreted with memcpy: a bit_cast of a vector
// element reads the wrong element with this compiler.)
__device__ __forceinline__ int bf16_max_bits(const u32x4& v) {
  const uint32_t w0 = v[0], w1 = v[1], w2 = v[2], w3 = v[3];
  s16x2 x0, x1, x2, x3;
  __builtin_memcpy(&x0, &w0, 4);
  __builtin_memcpy(&x1, &w1, 4);
  __builtin_memcpy(&x2, &w2, 4);
  __builtin_memcpy(&x3, &w3, 4);
  s16x2 a = __builtin_elementwise_max(__builtin_elementwise_max(x0, x1),
                                      __builtin_elementwise_max(x2, x3));
  return (int)a[0] > (int)a[1] ? (int)a[0] : (int)a[1];
}

__device__ __forceinline__ uint64_t block_max_key(uint64_t k, uint64_t* sred) {
  k = wave_max_u64(k);
  const int wave = threadIdx.x / kWave;
  if (lane_id() == 0) sred[wave] = k;
  __syncthreads();
  uint64_t r = sred[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) r = sred[w] > r ? sred[w] : r;
  __syncthreads();
  return r;
}

// Key of the largest non-NaN value among this lane's entries, lowest index
// on ties (0 if none).
template <int DT>
__device__ __forceinline__ uint64_t group_key(const u32x4& v, uint32_t i0) {
  using E = Elt<DT>;
  uint64_t k = 0ull;
#pragma unroll
  for (int e = 0; e < E::VN; ++e) {
    const float f = E::vget(v, e);
    const uint64_t ke = f == f ? make_key(f, i0 + e) : 0ull;
    k = ke > k ? ke : k;
  }
  return k;
}

// Row argmax partials.  Each wave keeps one running best (value, lowest
// index) key, the same in all its lanes, over interleaved 1 KB slices of the
// chunk; a 16-byte group is examined further only when it holds a value
// strictly larger than that best -- for bf16 and a positive best one packed
// signed 16-bit maximum decides it.  Slices of a wave are visited in
// increasing index order, so an equal value later never displaces the best.
// Work-group `bid` of rows * splits (kThreads threads): row bid / splits,
// chunk bid % splits; sred: kWaves words of LDS.
template <int DT>
__device__ __forceinline__ void argmax_part_body(const void* __restrict__ z, int64_t vocab, int splits,
                                                 int64_t chunk, uint64_t* __restrict__ part, int bid,
                                                 uint64_t* sred) {
  using E = Elt<DT>;
  const int64_t row = bid / splits;
  const int sp = bid % splits;
  const int64_t lo = (int64_t)sp * chunk, hi = lo + chunk < vocab ? lo + chunk : vocab;
  const void* rowp = (const char*)z + row * vocab * E::ESZ;
  const int wave = wave_id(), lane = lane_id();
  const unsigned mis = (unsigned)(size_t)((const char*)rowp + lo * E::ESZ) & 15u;
  const int64_t head = (int64_t)(((16u - mis) & 15u) / E::ESZ);
  const int64_t a0 = lo + head < hi ? lo + head : hi;
  const int64_t a1 = a0 + (hi - a0) / E::VN * E::VN;
  uint64_t best = 0ull;
  if (wave == 0) {  // head and tail outside 16-byte alignment, one per lane
    uint64_t k = 0ull;
    for (int64_t i = lo + lane; i < a0; i += kWave) {
      const float f = E::one(rowp, i);
      const uint64_t ke = f == f ? make_key(f, (uint32_t)i) : 0ull;
      k = ke > k ? ke : k;
    }
    for (int64_t i = a1 + lane; i < hi; i += kWave) {
      const float f = E::one(rowp, i);
      const uint64_t ke = f == f ? make_key(f, (uint32_t)i) : 0ull;
      k = ke > k ? ke : k;
    }
    best = uniform_u64(wave_max_u64(k));
  }
  const u32x4* vp = (const u32x4*)((const char*)rowp + a0 * E::ESZ);
  const int64_t ng = (a1 - a0) / E::VN;
  for (int64_t g0 = (int64_t)wave * kWave; g0 < ng; g0 += (int64_t)kThreads * kUnroll) {
    u32x4 v[kUnroll];
    bool ok[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t g = g0 + (int64_t)u * kThreads + lane;
      ok[u] = g < ng;
      v[u] = __builtin_nontemporal_load(vp + (ok[u] ? g : 0));
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const float bv = key_value(best);
      bool cand;
      if (DT == 1 && best != 0ull && bv > 0.f) {
        cand = (bf16_max_bits(v[u]) > (int)(__float_as_uint(bv) >> 16)) & ok[u];
      } else {
        float gm = E::vget(v[u], 0);
#pragma unroll
        for (int e = 1; e < E::VN; ++e) gm = fmaxf(gm, E::vget(v[u], e));
        cand = ((best == 0ull) | (gm > bv)) & ok[u];
      }
      if (ballot(cand) == 0ull) continue;
      const uint32_t i0 = (uint32_t)(a0 + (g0 + (int64_t)u * kThreads + lane) * E::VN);
      const uint64_t k = wave_max_u64(cand ? group_key<DT>(v[u], i0) : 0ull);
      best = uniform_u64(k > best ? k : best);
    }
  }
  best = block_max_key(best, sred);
  if (threadIdx.x == 0) part[row * splits + sp] = best;
}

// one wave per request: merge the argmax partials of rows t = 0..T, then the
// longest agreeing prefix
// (one wave: lanes 0..63 of the caller's first wave)
__device__ __forceinline__ void greedy_final_body(const uint64_t* __restrict__ part, int splits, int T,
                                                  const int32_t* __restrict__ path_tok,
                                                  int32_t* __restrict__ accept_len, int32_t* __restrict__ out_tok,
                                                  int b) {
  const int lane = lane_id();
  // the drafted token of this lane's position, requested with the keys
  const int32_t pt = path_tok[(int64_t)b * T + (lane < T ? lane : 0)];
  int y = -1;
  if (lane <= T) {
    const uint64_t* p = part + ((int64_t)b * (T + 1) + lane) * splits;
    uint64_t k = 0;
#pragma unroll 8
    for (int s = 0; s < splits; ++s) k = p[s] > k ? p[s] : k;
    y = k ? (int)key_index(k) : -1;
  }
  bool miss = lane < T && pt != y;
  uint64_t mm = ballot(miss);
  int n = mm ? __ffsll((unsigned long long)mm) - 1 : T;
  int yn = __shfl(y, n);
  if (lane == 0) accept_len[b] = n;
  if (lane <= T) {
    int v = lane < n ? pt : lane == n ? yn : -1;
    out_tok[(int64_t)b * (T + 1) + lane] = v;
  }
}

}  // namespace verifyd
}  // namespace df2

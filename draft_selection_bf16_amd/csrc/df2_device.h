// df2_device.h -- device-side helpers shared by the HIP kernels of the
// draft-block library (gfx950, wave64).  Internal; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace df2 {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// word 3 of a raw (untyped, stride 0) buffer resource on gfx9-family GPUs
constexpr int kBufferWord3 = 0x00020000;

// ---------------------------------------------------------------- elements
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ float half_to_f32(uint16_t h) {
  _Float16 v;
  __builtin_memcpy(&v, &h, sizeof v);
  return (float)v;
}

// float -> bf16 bits, round to nearest even (inputs here are finite)
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---------------------------------------------------------------- ordering
// Order-preserving unsigned code of a float.  -0 is folded onto +0 so that
// equal values compare equal.
__device__ __forceinline__ uint32_t ord_of(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float value_of_ord(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}
// A (value, index) pair as one integer: larger value first, and among equal
// values the lower index first.  Distinct indices give distinct keys, so a
// top-K by key is unique and independent of the order of any merge.  Key 0
// is never produced for a finite value and serves as "empty".
__device__ __forceinline__ uint64_t make_key(float f, uint32_t idx) {
  return ((uint64_t)ord_of(f) << 32) | (uint64_t)(~idx);
}
__device__ __forceinline__ uint32_t key_index(uint64_t k) { return ~(uint32_t)k; }
__device__ __forceinline__ float key_value(uint64_t k) { return value_of_ord((uint32_t)(k >> 32)); }

// Online-softmax partial of a set of logits: key = make_key of its maximum
// (value, lowest index), s = sum of exp2((z - value(key)) c).  Combine two
// partials (key 0 = empty), the sum kept relative to the larger maximum.
__device__ __forceinline__ void combine_part(uint64_t& k, float& s, uint64_t k2, float s2, float c) {
  if (k2 == 0ull) return;
  if (k == 0ull) {
    k = k2;
    s = s2;
    return;
  }
  float m1 = key_value(k), m2 = key_value(k2);
  if (k2 > k) {
    s = s * exp2f((m1 - m2) * c) + s2;
    k = k2;
  } else {
    s = s + s2 * exp2f((m2 - m1) * c);
  }
}

// ---------------------------------------------------------------- wave ops
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  lo = __shfl_xor(lo, m);
  hi = __shfl_xor(hi, m);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src) {
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  lo = __shfl(lo, src);
  hi = __shfl(hi, src);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    uint64_t o = shfl_xor_u64(v, m);
    v = o > v ? o : v;
  }
  return v;
}
__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}
__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}
__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }
// index of this wave in its work-group, in a scalar register
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave)); }
// a value that is the same in every lane, moved to scalar registers so that
// branches on it are scalar branches
__device__ __forceinline__ uint64_t uniform_u64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }
// number of set bits of m below this lane
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return __popcll(m & ((1ull << lane_id()) - 1ull));
}

// The 16th largest of the non-empty keys held PER to a lane (keys are
// unique), or 0 when there are fewer than 16.  MSB-first bit search: keep a
// bit when at least 16 keys are >= the prefix with that bit set.  Counts are
// ballot popcounts, so the search runs on the scalar unit with no cross-lane
// data movement.
template <int PER>
__device__ __forceinline__ uint64_t kth16(const uint64_t (&keys)[PER]) {
  uint64_t t = 0;
#pragma unroll 4
  for (int bit = 63; bit >= 0; --bit) {
    const uint64_t cand = t | (1ull << bit);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) cnt += __popcll(ballot(keys[i] >= cand));
    if (cnt >= 16) t = cand;
  }
  return t;
}

// Move the keys >= t (non-empty) of every lane to dst[0..n) (in no
// particular order) and return n.  dst may alias the source buffer only if
// the keys were already loaded to registers.
template <int PER>
__device__ __forceinline__ int gather_at_least(const uint64_t (&keys)[PER], uint64_t t,
                                               uint64_t* dst) {
  int n = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const bool keep = keys[i] != 0ull && keys[i] >= t;
    const uint64_t m = ballot(keep);
    if (keep) dst[n + lanes_below(m)] = keys[i];
    n += __popcll(m);
  }
  return n;
}

// Number of the wave's 64 keys (one per lane) that are larger than this
// lane's (keys distinct or 0).  64 independent compares against values read
// from each lane -- no ballot/popcount round trips on the critical path.
__device__ __forceinline__ int rank_in_wave(uint64_t key) {
  const uint32_t lo = (uint32_t)key, hi = (uint32_t)(key >> 32);
  int r = 0;
#pragma unroll 16
  for (int i = 0; i < kWave; ++i) {
    // (readlane returns int: widen through uint32_t, not by sign extension)
    const uint64_t o = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(hi, i) << 32) |
                       (uint64_t)(uint32_t)__builtin_amdgcn_readlane(lo, i);
    r += o > key ? 1 : 0;
  }
  return r;
}

// Number of the N keys keys[0..N) (LDS, N even) that are larger than `key`.
// All lanes read the same addresses (broadcast LDS reads), so the loads
// pipeline and the compares are independent.
template <int N>
__device__ __forceinline__ int rank_in_lds(uint64_t key, const uint64_t* keys) {
  typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));
  int r = 0;
#pragma unroll 16
  for (int i = 0; i < N; i += 2) {
    const u64x2 o = *(const u64x2*)(keys + i);
    r += (o[0] > key ? 1 : 0) + (o[1] > key ? 1 : 0);
  }
  return r;
}

// Exclusive prefix over the lanes of a small count c (0 <= c < 16) and the
// wave total, from one ballot per bit of c (independent ballots).
__device__ __forceinline__ int lane_prefix16(int c, int& total) {
  int ex = 0, tot = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const uint64_t m = ballot((c >> b) & 1);
    ex += lanes_below(m) << b;
    tot += __popcll(m) << b;
  }
  total = tot;
  return ex;
}

// buf[0..n) holds n <= 16 distinct keys (LDS, this wave's own); lane j < n
// returns the j-th largest, other lanes 0.  Each key's rank is the number of
// larger keys; keys are scattered to their ranks in the same buffer.
__device__ __forceinline__ uint64_t sorted16(uint64_t* buf, int n) {
  const int lane = lane_id();
  const uint64_t mine = lane < n ? buf[lane] : 0ull;
  int rank = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i)
    if (i < n) rank += buf[i] > mine ? 1 : 0;
  __builtin_amdgcn_wave_barrier();
  if (lane < n) buf[rank] = mine;
  __builtin_amdgcn_wave_barrier();
  return lane < n ? buf[lane] : 0ull;
}

// ---------------------------------------------------------------- Philox
// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds; each
// multiplies counter words 0 and 2 by the round multipliers, and xors the
// high product halves with words 1/3 and the round key; the key advances by
// the Weyl increments between rounds.
struct u64x4 {
  uint64_t w[4];
};
__device__ __forceinline__ u64x4 philox4x64_10(uint64_t key0, uint64_t key1, uint64_t c0,
                                               uint64_t c1, uint64_t c2, uint64_t c3) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    uint64_t lo0 = M0 * c0, hi0 = __umul64hi(M0, c0);
    uint64_t lo1 = M1 * c2, hi1 = __umul64hi(M1, c2);
    uint64_t n0 = hi1 ^ c1 ^ key0, n2 = hi0 ^ c3 ^ key1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
    key0 += W0;
    key1 += W1;
  }
  u64x4 o;
  o.w[0] = c0;
  o.w[1] = c1;
  o.w[2] = c2;
  o.w[3] = c3;
  return o;
}
// (2 * (w >> 41) + 1) * 2^-24: exact in fp32, inside (0, 1)
__device__ __forceinline__ float uniform_of_word(uint64_t w) {
  return (float)(2u * (uint32_t)(w >> 41) + 1u) * (1.0f / 16777216.0f);
}
__device__ __forceinline__ float cycle_uniform(uint64_t seed, int b, int t, int word) {
  u64x4 o = philox4x64_10(seed, 0, (uint64_t)t, (uint64_t)b, 0, 0);
  return uniform_of_word(o.w[word]);
}

}  // namespace df2

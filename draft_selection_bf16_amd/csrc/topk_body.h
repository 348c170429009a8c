// topk_body.h -- device code of the row top-K (topk.hip): the chunk scan
// and selection of one work-group and the per-row merge of the chunks'
// lists, as device functions that take their block index and LDS from the
// caller (the stand-alone kernels in topk.hip, or a persistent kernel).
// Internal; not part of the ABI.
#pragma once

#include "df2_device.h"

namespace df2 {
namespace topkd {


constexpr int kCap = 256;        // LDS keys per wave
constexpr int kPer = kCap / kWave;
constexpr int kUnroll = 4;       // 16-byte loads in flight per lane
constexpr int kQueue = 320;      // queued 16-byte groups per wave
constexpr int kQueueFlush = kQueue - kUnroll * kWave;   // expand above this

typedef short s16x2 __attribute__((ext_vector_type(2)));

// Element access of a 16-byte group: get0 reads element 0, shift drops it
// (the next element moves to position 0), raw/nan build groups from
// scalar loads.
template <typename E>
struct Vec;
template <>
struct Vec<float> {               // fp32: 4 per 16 bytes
  static constexpr int n = 4;
  static constexpr int value_bits = 32;   // bits of the order key that vary
  __device__ static float get0(const u32x4& v) { return __uint_as_float(v[0]); }
  __device__ static u32x4 shift(const u32x4& v) { return u32x4{v[1], v[2], v[3], 0u}; }
  __device__ static float get(const u32x4& v, int e) { return __uint_as_float(v[e]); }
  __device__ static uint32_t raw(const void* p, int64_t i) { return ((const uint32_t*)p)[i]; }
  static constexpr uint32_t nan = 0x7fc00000u;
};
struct Bf16 {};
struct F16 {};
template <typename H>
struct Vec16 {                    // 16-bit types: 8 per 16 bytes
  static constexpr int n = 8;
  __device__ static u32x4 shift(const u32x4& v) {
    return u32x4{__builtin_amdgcn_alignbit(v[1], v[0], 16), __builtin_amdgcn_alignbit(v[2], v[1], 16),
                 __builtin_amdgcn_alignbit(v[3], v[2], 16), v[3] >> 16};
  }
  __device__ static uint32_t raw(const void* p, int64_t i) { return ((const uint16_t*)p)[i]; }
};
template <>
struct Vec<Bf16> : Vec16<Bf16> {
  static constexpr int value_bits = 16;
  static constexpr uint32_t nan = 0x7fc0u;
  __device__ static float get0(const u32x4& v) { return bf16_lo(v[0]); }
  __device__ static float get(const u32x4& v, int e) {
    uint32_t w = v[e >> 1];
    return (e & 1) ? bf16_hi(w) : bf16_lo(w);
  }
};
template <>
struct Vec<F16> : Vec16<F16> {
  static constexpr int value_bits = 32;
  static constexpr uint32_t nan = 0x7e00u;
  __device__ static float get0(const u32x4& v) { return half_to_f32((uint16_t)(v[0] & 0xffffu)); }
  __device__ static float get(const u32x4& v, int e) {
    uint32_t w = v[e >> 1];
    return half_to_f32((uint16_t)((e & 1) ? (w >> 16) : (w & 0xffffu)));
  }
};

// The group of entries i0 .. i0 + n - 1 of a row, those outside [lo, hi)
// replaced by NaN (never a candidate).
template <typename E>
__device__ __forceinline__ u32x4 partial_group(const void* rowp, int64_t i0, int64_t lo, int64_t hi) {
  constexpr int VN = Vec<E>::n, PW = VN / 4;   // elements per 32-bit word
  u32x4 r;
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < PW; ++j) {
      const int64_t i = i0 + h * PW + j;
      const uint32_t b = (i >= lo && i < hi) ? Vec<E>::raw(rowp, i) : Vec<E>::nan;
      w |= b << (32 / PW * j);
    }
    r[h] = w;
  }
  return r;
}

// Per-wave filter state.  `buf` is this wave's LDS key buffer, `q`/`qi` its
// queue of 16-byte groups (raw data and index of the first element) that
// may hold a candidate; `share` holds one published threshold per wave of
// the work-group.
struct Filter {
  uint64_t* buf;
  u32x4* q;
  uint32_t* qi;
  float* share;   // read and written with relaxed work-group atomics
  uint32_t* prime; // the work-group's lane maxima of the first batch
  int cnt;     // keys in buf
  int qn;      // groups in q
  float thr;   // entries with value < thr cannot be in the result
};

__device__ __forceinline__ void publish(Filter& F, int wave) {
  __hip_atomic_store(F.share + wave, F.thr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Largest t (with the low 32 - VB bits zero) such that at least 16 of the
// order values held N to a lane are >= t (0 stands for "none"); 0 if fewer
// than 16.  Keys with ord >= t are a superset of the 16 best (ties at the
// boundary are kept).
template <int VB, int N>
__device__ __forceinline__ uint32_t value_cut16(const uint32_t (&ord)[N]) {
  uint32_t t = 0;
#pragma unroll 4
  for (int bit = 31; bit >= 32 - VB; --bit) {
    const uint32_t cand = t | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < N; ++i) cnt += __popcll(ballot(ord[i] >= cand));
    if (cnt >= 16) t = cand;
  }
  return t;
}

// Cut the buffer back to the keys whose value can still be among the 16
// best; publish and raise the threshold.  Falls back to the exact 64-bit cut
// when ties at the boundary would leave the buffer nearly full.
template <int VB>
__device__ __forceinline__ void compact(Filter& F, int wave) {
  uint64_t keys[kPer];
  uint32_t ord[kPer];
  const int lane = lane_id();
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    int s = lane + i * kWave;
    keys[i] = s < F.cnt ? F.buf[s] : 0ull;
    ord[i] = (uint32_t)(keys[i] >> 32);
  }
  __builtin_amdgcn_wave_barrier();
  const uint32_t t = value_cut16<VB, kPer>(ord);
  int n = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) n += __popcll(ballot(keys[i] != 0ull && ord[i] >= t));
  const uint64_t tk = n > kCap - 2 * kWave ? kth16<kPer>(keys)   // massive ties: exact cut
                                           : (uint64_t)t << 32;
  F.cnt = gather_at_least<kPer>(keys, tk, F.buf);
  if (t != 0u) {
    const float v = value_of_ord(t);
    if (v > F.thr) F.thr = v;
    if (lane == 0) publish(F, wave);
  }
  __builtin_amdgcn_wave_barrier();
}

template <int NW>
__device__ __forceinline__ void refresh(Filter& F) {
  float t = F.thr;
#pragma unroll
  for (int w = 0; w < NW; ++w)
    t = fmaxf(t, __hip_atomic_load(F.share + w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
  // the same value in every lane: keep it in a scalar register
  F.thr = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(t)));
}

// Expand the queued groups into keys, one group per lane: each lane counts
// the entries of its group that reach the threshold, a prefix over the
// counts gives every lane its slots, and the keys are written in one go.
// (When they would overflow the buffer, it is cut back first; if they still
// would, the round goes element by element with a cut whenever needed.)
// Then the buffer is cut back to at most about `keep` keys, which raises the
// threshold to the 16th best value seen so far.
template <typename E>
__device__ __forceinline__ void flush(Filter& F, int wave, int keep) {
  constexpr int VB = Vec<E>::value_bits;
  constexpr int VN = Vec<E>::n;
  const int lane = lane_id();
  for (int base = 0; base < F.qn; base += kWave) {
    const int s = base + lane;
    const bool valid = s < F.qn;
    const u32x4 v = F.q[valid ? s : 0];
    const uint32_t i0 = F.qi[valid ? s : 0];
    __builtin_amdgcn_wave_barrier();
    float f[VN];
#pragma unroll
    for (int e = 0; e < VN; ++e) f[e] = Vec<E>::get(v, e);
    int c = 0;
#pragma unroll
    for (int e = 0; e < VN; ++e) c += (valid && f[e] >= F.thr) ? 1 : 0;
    int total;
    int ex = lane_prefix16(c, total);
    if (F.cnt + total > kCap) {
      compact<VB>(F, wave);
      c = 0;
#pragma unroll
      for (int e = 0; e < VN; ++e) c += (valid && f[e] >= F.thr) ? 1 : 0;
      ex = lane_prefix16(c, total);
    }
    if (F.cnt + total <= kCap) {
      int slot = F.cnt + ex;
#pragma unroll
      for (int e = 0; e < VN; ++e)
        if (valid && f[e] >= F.thr) F.buf[slot++] = make_key(f[e], i0 + e);
      F.cnt += total;
      __builtin_amdgcn_wave_barrier();
    } else {
#pragma unroll 1
      for (int e = 0; e < VN; ++e) {
        bool pass = valid && f[e] >= F.thr;
        uint64_t m = ballot(pass);
        if (m == 0ull) continue;
        if (F.cnt + __popcll(m) > kCap) {
          compact<VB>(F, wave);
          pass = valid && f[e] >= F.thr;
          m = ballot(pass);
        }
        if (pass) F.buf[F.cnt + lanes_below(m)] = make_key(f[e], i0 + e);
        F.cnt += __popcll(m);
        __builtin_amdgcn_wave_barrier();
      }
    }
  }
  F.qn = 0;
  if (F.cnt > keep) compact<VB>(F, wave);
}

// Could any of the eight bf16 values of v reach thr (> 0)?  Positive bf16
// values order like their bits read as signed 16-bit integers, and every
// negative value (and -0) reads as negative: one packed maximum decides.
// (The words are reinterpreted with memcpy: a bit_cast of a vector element
// reads the wrong element with this compiler.)
__device__ __forceinline__ bool bf16_may_pass(const u32x4& v, int thr16) {
  const uint32_t w0 = v[0], w1 = v[1], w2 = v[2], w3 = v[3];
  s16x2 x0, x1, x2, x3;
  __builtin_memcpy(&x0, &w0, 4);
  __builtin_memcpy(&x1, &w1, 4);
  __builtin_memcpy(&x2, &w2, 4);
  __builtin_memcpy(&x3, &w3, 4);
  s16x2 a = __builtin_elementwise_max(__builtin_elementwise_max(x0, x1),
                                      __builtin_elementwise_max(x2, x3));
  const int m = (int)a[0] > (int)a[1] ? (int)a[0] : (int)a[1];
  return m >= thr16;
}

// Filter the entries [lo, hi) of a row into the waves' key buffers.  Every
// wave of the work-group calls it (it holds one work-group barrier).
template <typename E, int NW>
__device__ __forceinline__ void scan_range(Filter& F, const void* rowp, int64_t lo, int64_t hi,
                                           int wave) {
  constexpr int VN = Vec<E>::n;
  constexpr int VB = Vec<E>::value_bits;
  constexpr bool kBf16 = VB == 16;
  const int lane = lane_id();
  const int esz = sizeof(u32x4) / VN;
  // the body [a0, a1) is 16-byte aligned; the head [lo, a0) and the tail
  // [a1, hi) have fewer than VN entries each and go to wave 0's queue as
  // NaN-padded groups (pointer arithmetic stays on typed pointers so that
  // loads remain global loads)
  int64_t a0, a1;
  {
    const unsigned mis = (unsigned)(size_t)((const char*)rowp + lo * esz) & 15u;
    int64_t head = (int64_t)(((16u - mis) & 15u) / esz);
    a0 = lo + head < hi ? lo + head : hi;
    a1 = a0 + (hi - a0) / VN * VN;
  }
  if (wave == 0) {
    const bool c = (lane == 0 && a0 > lo) || (lane == 1 && hi > a1);
    const uint64_t m = ballot(c);
    if (c) {
      const int64_t i0 = lane == 0 ? lo : a1;
      F.q[lanes_below(m)] = partial_group<E>(rowp, i0, lo, lane == 0 ? a0 : hi);
      F.qi[lanes_below(m)] = (uint32_t)i0;
    }
    F.qn = __popcll(m);
    __builtin_amdgcn_wave_barrier();
  }
  const u32x4* vp = (const u32x4*)((const char*)rowp + a0 * esz);
  const int64_t ngroups = (a1 - a0) / VN;   // 16-byte groups
  const int64_t stride = (int64_t)NW * kWave;
  const int ng = (int)ngroups;   // < 2^31: rows hold < 2^32 entries
  // Software-pipelined over two register sets: the loads of the next
  // iteration are issued before this one's groups are tested (no register
  // copy, which would wait for the loads), so two iterations' loads (8 KB
  // per wave) are in flight.
  const int step = (int)stride * kUnroll;
  auto load = [&](int g0, u32x4 (&v)[kUnroll], bool (&ok)[kUnroll]) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int g = g0 + u * (int)stride + lane;
      ok[u] = g < ng;
      v[u] = __builtin_nontemporal_load(vp + (ok[u] ? g : 0));
    }
  };
  auto process = [&](int g0, const u32x4 (&v)[kUnroll], const bool (&ok)[kUnroll]) {
    if (F.qn > kQueueFlush) flush<E>(F, wave, 32);
    // the threshold is the same in all lanes: decide the test once per
    // iteration, on the scalar unit
    const float thr = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(F.thr)));
    uint64_t m[kUnroll];
    if (kBf16 && thr > 0.f) {
      const int thr16 = (int)(__float_as_uint(thr) >> 16);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) m[u] = ballot(bf16_may_pass(v[u], thr16) & ok[u]);
    } else {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        float gm = Vec<E>::get(v[u], 0);
#pragma unroll
        for (int e = 1; e < VN; ++e) gm = fmaxf(gm, Vec<E>::get(v[u], e));
        m[u] = ballot((gm >= thr) & ok[u]);
      }
    }
    // queue the groups that may hold a candidate (rare once the threshold
    // is up); flush() expands them in bulk
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (m[u] == 0ull) continue;
      if ((m[u] >> lane) & 1ull) {
        const int s = F.qn + lanes_below(m[u]);
        F.q[s] = v[u];
        F.qi[s] = (uint32_t)(a0 + (int64_t)(g0 + u * (int)stride + lane) * VN);
      }
      F.qn += __popcll(m[u]);
      __builtin_amdgcn_wave_barrier();
    }
    refresh<NW>(F);
  };
  u32x4 va[kUnroll], vb[kUnroll];
  bool oka[kUnroll], okb[kUnroll];
  int g0 = wave * kWave;
  uint32_t lmax = 0u;
  if (g0 < ng) {
    load(g0, va, oka);
    // prime the threshold from the batch just issued (kUnroll groups per
    // lane): each lane's maximum; below, the 16th largest of the work-
    // group's lane maxima, which 16 distinct entries reach (NaN never
    // qualifies); the scan sees these entries again below.  With kUnroll x
    // VN = 32 bf16 entries per lane, one wave's 16th largest of 64 sits near
    // the 99th percentile of a row's values (against the 97th for the 16th
    // best of one group per lane: at 480 rows of 151,936 a wave then queued
    // 138 groups and flushed 1.14 times in its scan, 6,500 cycles a flush;
    // with it 80 groups and 0.99 flushes), the work-group's 16th largest of
    // 512 near the 99.9th: top-k 31.9 -> 31.55 us at 480 rows, batch 8 /
    // block 16 72.4 -> 71.1 us and batch 32 / block 8 85.4 -> 84.2 us per
    // cycle (the stress cycle 812.5 -> 814.8).
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int e = 0; e < VN; ++e) {
        const float f = Vec<E>::get(va[u], e);
        const uint32_t o = oka[u] && f == f ? ord_of(f) : 0u;
        lmax = o > lmax ? o : lmax;
      }
  }
  F.prime[wave * kWave + lane] = lmax;
  __syncthreads();
  {
    uint32_t lm[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) lm[w] = F.prime[w * kWave + lane];
    const uint32_t t = value_cut16<VB, NW>(lm);
    if (t != 0u) {
      F.thr = fmaxf(F.thr, value_of_ord(t));
      if (lane == 0) publish(F, wave);
    }
  }
  while (g0 < ng) {   // the same in all lanes
    if (g0 + step < ng) load(g0 + step, vb, okb);
    process(g0, va, oka);
    g0 += step;
    if (g0 >= ng) break;
    if (g0 + step < ng) load(g0 + step, va, oka);
    process(g0, vb, okb);
    g0 += step;
  }
}

// LDS of one (row, chunk) work-group of NW waves.
// Rank the ns <= kThreads pooled keys ssurv[0..ns) (distinct) and put the 16
// best in sbest[0..16) (slots past ns keep 0); ends with a work-group
// barrier.  rank = number of larger keys: the list is padded with empty
// keys to a multiple of 16; P = kThreads / n16 threads share a key, each
// counting the larger keys in its 1/P of the list (two keys per LDS load,
// eight loads in flight), the counts meeting in LDS.
template <int kThreads>
__device__ __forceinline__ void rank_pool(uint64_t* ssurv, int* srank, int ns, uint64_t* sbest) {
  const int tid = threadIdx.x;
  const int n16 = (ns + 15) & ~15;
  if (tid < n16 - ns) ssurv[ns + tid] = 0ull;
  srank[tid] = 0;
  __syncthreads();
  const int P = n16 > 0 ? kThreads / n16 : 1;   // >= 1
  const int len = n16 / P > 16 ? ((n16 / P) + 15) & ~15 : 16;   // parts past n16 count nothing
  const int part = tid / (n16 > 0 ? n16 : 1), i = tid - part * n16;
  uint64_t key = 0ull;
  if (part < P && i < ns) {
    key = ssurv[i];
    typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));
    const int j1 = (part + 1) * len < n16 ? (part + 1) * len : n16;
    int c = 0;
    for (int j = part * len; j < j1; j += 16) {
      u64x2 o[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) o[u] = *(const u64x2*)(ssurv + j + 2 * u);
#pragma unroll
      for (int u = 0; u < 8; ++u) c += (o[u][0] > key ? 1 : 0) + (o[u][1] > key ? 1 : 0);
    }
    if (c > 0) atomicAdd(&srank[i], c);
  }
  __syncthreads();
  key = tid < ns ? ssurv[tid] : 0ull;
  const int r = tid < ns ? srank[tid] : kThreads;
  if (key != 0ull && r < 16) sbest[r] = key;
  __syncthreads();
}

// Wave 0: the 16 best of the NW waves' lists smerge[w * 16 .. + 16) into
// sbest (by rank: every key's number of larger keys).
template <int NW>
__device__ __forceinline__ void merge_wave_lists(const uint64_t* smerge, uint64_t* sbest, int lane) {
  static_assert(NW % 4 == 0, "whole lanes of candidates");
#pragma unroll
  for (int c = 0; c < NW / 4; ++c) {
    const uint64_t kc = smerge[c * kWave + lane];
    const int rc = rank_in_lds<NW * 16>(kc, smerge);
    if (kc != 0ull && rc < 16) sbest[rc] = kc;
  }
  __builtin_amdgcn_wave_barrier();
}

// Wave 0: the chunk's result -- the final k (index, value) pairs of the row
// with one chunk per row, else the chunk's 16 keys for the merge.
__device__ __forceinline__ void write_chunk_result(const uint64_t* sbest, int splits, int k, int64_t row,
                                                   int split, int32_t* out_idx, float* out_val, uint64_t* part,
                                                   int lane) {
  if (splits == 1) {
    if (lane < k) {
      const uint64_t key = sbest[lane];
      out_idx[row * k + lane] = (int32_t)key_index(key);
      out_val[row * k + lane] = key_value(key);
    }
  } else if (lane < 16) {
    part[((int64_t)row * splits + split) * 16 + lane] = sbest[lane];
  }
}

template <int NW>
struct TopkChunkLds {
  __attribute__((aligned(16))) uint64_t sbuf[NW][kCap];
  u32x4 squeue[NW][kQueue];
  uint32_t sqidx[NW][kQueue];
  __attribute__((aligned(16))) uint64_t smerge[NW * 16];
  float sthr[NW];
  uint32_t sprime[NW * kWave];
  __attribute__((aligned(16))) uint64_t ssurv[NW * kWave + 16];
  int srank[NW * kWave];
  int snsurv;
  uint64_t sbest[16];
  uint64_t s2nd[NW];
};

// Work-group `bid` of rows * splits work-groups of NW waves: row bid /
// splits, chunk bid % splits.  If splits == 1 writes the final k results,
// else the 16 best keys of the chunk to part.  Waves other than 0 may
// return before the end (no work-group barrier follows their return).
template <typename E, int NW>
__device__ __forceinline__ void topk_chunk_body(const void* __restrict__ logits, int64_t vocab, int splits,
                                                int64_t chunk, int k, int32_t* __restrict__ out_idx,
                                                float* __restrict__ out_val, uint64_t* __restrict__ part, int bid,
                                                TopkChunkLds<NW>& L) {
  constexpr int kThreads = NW * kWave;
  auto& sbuf = L.sbuf;
  auto& squeue = L.squeue;
  auto& sqidx = L.sqidx;
  auto& smerge = L.smerge;
  auto& sthr = L.sthr;
  const int wave = wave_id(), lane = lane_id();
  const int64_t row = bid / splits;
  const int split = bid % splits;
  const int64_t lo = (int64_t)split * chunk;
  const int64_t hi = lo + chunk < vocab ? lo + chunk : vocab;
  const int esz = sizeof(u32x4) / Vec<E>::n;
  const void* rowp = (const char*)logits + row * vocab * esz;

  if (lane == 0) sthr[wave] = -INFINITY;
  __syncthreads();
  Filter F{sbuf[wave], squeue[wave], sqidx[wave], sthr, L.sprime, 0, 0, -INFINITY};
  scan_range<E, NW>(F, rowp, lo, hi, wave);
  // Keep up to 64 keys per wave (no final cut), then filter every wave's
  // keys by two lower bounds on the chunk's 16th best key: the largest
  // published threshold (a value some wave saw at least 16 keys reach) and
  // the smallest of the waves' (16 / NW)-th best keys (with 8 waves their
  // second best).  The 16 best all pass; a few dozen keys survive at
  // V = 151,936.  Survivors are ranked against each other by all threads.
  // With massive ties (more survivors than threads) every wave first takes
  // its own 16 best and wave 0 merges the NW x 16.
  flush<E>(F, wave, kWave);
  if (lane == 0) publish(F, wave);
  auto& ssurv = L.ssurv;
  auto& srank = L.srank;
  int& snsurv = L.snsurv;
  auto& sbest = L.sbest;
  auto& s2nd = L.s2nd;
  uint64_t keys[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int s2 = lane + i * kWave;
    keys[i] = s2 < F.cnt ? F.buf[s2] : 0ull;
  }
  {
    // this wave's (16 / NW)-th largest key (0 if it holds fewer): the NW
    // waves' best 16 / NW keys are 16 distinct keys at least as large as
    // the smallest of these
    static_assert(16 % NW == 0, "16 / NW keys per wave");
    uint64_t m = ~0ull;
#pragma unroll
    for (int j = 0; j < 16 / NW; ++j) {
      uint64_t c = 0ull;   // keys are distinct: the largest below the previous one
#pragma unroll
      for (int i = 0; i < kPer; ++i) c = (keys[i] < m && keys[i] > c) ? keys[i] : c;
      m = wave_max_u64(c);
    }
    if (lane == 0) s2nd[wave] = m;
  }
  if (threadIdx.x == 0) snsurv = 0;
  if (threadIdx.x < 16) sbest[threadIdx.x] = 0ull;
  __syncthreads();
  {
    float g = -INFINITY;
    uint64_t kb = ~0ull;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      g = fmaxf(g, __hip_atomic_load(F.share + w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
      kb = s2nd[w] < kb ? s2nd[w] : kb;
    }
    const uint32_t go = ord_of(g);
    bool keep[kPer];
    int n = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      keep[i] = keys[i] != 0ull && (uint32_t)(keys[i] >> 32) >= go && keys[i] >= kb;
      n += __popcll(ballot(keep[i]));
    }
    int base = 0;
    if (lane == 0 && n > 0) base = atomicAdd(&snsurv, n);
    base = __builtin_amdgcn_readfirstlane(base);
    if (base + n <= kThreads) {
      int off = base;
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const uint64_t m = ballot(keep[i]);
        if (keep[i]) ssurv[off + lanes_below(m)] = keys[i];
        off += __popcll(m);
      }
    }
  }
  __syncthreads();
  const int ns = snsurv;   // the same in every wave
  if (ns <= kThreads) {
    rank_pool<kThreads>(ssurv, srank, ns, sbest);
    if (wave != 0) return;
  } else {
    // The 16 best keys of this wave: normally at most 64 keys are left, and
    // each one's rank among them is its place; with many ties at the cut, an
    // exact 64-bit search first.
    uint64_t* mine16 = smerge + wave * 16;
    if (lane < 16) mine16[lane] = 0ull;
    __builtin_amdgcn_wave_barrier();
    if (F.cnt <= kWave) {
      const uint64_t key = lane < F.cnt ? F.buf[lane] : 0ull;
      if (lane >= F.cnt) F.buf[lane] = 0ull;   // pad to 64 keys
      __builtin_amdgcn_wave_barrier();
      const int r = rank_in_lds<kWave>(key, F.buf);
      if (key != 0ull && r < 16) mine16[r] = key;
    } else {
      uint64_t keys[kPer];
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        int s2 = lane + i * kWave;
        keys[i] = s2 < F.cnt ? F.buf[s2] : 0ull;
      }
      __builtin_amdgcn_wave_barrier();
      const uint64_t t = kth16<kPer>(keys);
      gather_at_least<kPer>(keys, t, mine16);   // exactly 16 keys (all distinct)
    }
    __syncthreads();
    if (wave != 0) return;
    // wave 0: the 16 best of the NW x 16 candidates (NW / 4 per lane), by rank
    merge_wave_lists<NW>(smerge, sbest, lane);
  }
  write_chunk_result(sbest, splits, k, row, split, out_idx, out_val, part, lane);
}

// ---- short chunks (at most kThreads * EPT entries) ----------------------
// With few rows every row is cut into many short chunks, and the streaming
// filter above (priming, queues, compaction) costs more than the chunk's
// one round of loads.  Here every thread loads its EPT entries at once
// (entry e of thread t is lo + e * kThreads + t, so each load instruction
// of a wave reads 64 consecutive entries), and
//  * each wave takes as its bound the 16th largest of its lanes' maxima:
//    16 lanes hold an entry at least that large, so the wave -- and the
//    work-group -- has 16 entries at or above it;
//  * the work-group's bound is the largest of the waves' bounds; the entries
//    that reach it (a few dozen on these rows) are pooled in LDS and ranked
//    as in the long path;
//  * more than kThreads of them (massive ties) falls back to the exact
//    per-wave 64-bit search and the merge of the NW x 16.
template <int NW>
struct TopkSmallLds {
  __attribute__((aligned(16))) uint64_t ssurv[NW * kWave + 16];
  int srank[NW * kWave];
  __attribute__((aligned(16))) uint64_t smerge[NW * 16];
  uint32_t swb[NW];
  int snsurv;
  uint64_t sbest[16];
};

template <typename E, int NW, int EPT>
__device__ __forceinline__ void topk_small_body(const void* __restrict__ logits, int64_t vocab, int splits,
                                                int64_t chunk, int k, int32_t* __restrict__ out_idx,
                                                float* __restrict__ out_val, uint64_t* __restrict__ part, int bid,
                                                TopkSmallLds<NW>& L) {
  constexpr int kThreads = NW * kWave;
  constexpr int VB = Vec<E>::value_bits;
  const int wave = wave_id(), lane = lane_id(), tid = threadIdx.x;
  const int64_t row = bid / splits;
  const int split = bid % splits;
  const int64_t lo = (int64_t)split * chunk;
  const int64_t hi = lo + chunk < vocab ? lo + chunk : vocab;   // lo < hi
  const int esz = sizeof(u32x4) / Vec<E>::n;
  const void* rowp = (const char*)logits + row * vocab * esz;
  // every load unconditional (clamped into the chunk), so all are in flight
  uint32_t raw[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int64_t i = lo + (int64_t)e * kThreads + tid;
    raw[e] = Vec<E>::raw(rowp, i < hi ? i : hi - 1);
  }
  if (tid == 0) L.snsurv = 0;
  if (tid < 16) L.sbest[tid] = 0ull;
  // order values (0: outside the chunk or NaN, never a candidate)
  uint32_t ord[EPT];
  uint32_t lmax = 0u;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const float f = Vec<E>::get0(u32x4{raw[e], 0u, 0u, 0u});
    const bool ok = lo + (int64_t)e * kThreads + tid < hi && f == f;
    ord[e] = ok ? ord_of(f) : 0u;   // a number's order value is never 0
    lmax = ord[e] > lmax ? ord[e] : lmax;
  }
  const uint32_t lm[1] = {lmax};
  const uint32_t wb = value_cut16<VB, 1>(lm);   // 0: fewer than 16 lanes hold a number
  if (lane == 0) L.swb[wave] = wb;
  __syncthreads();
  uint32_t bound = 0u;
#pragma unroll
  for (int w = 0; w < NW; ++w) bound = L.swb[w] > bound ? L.swb[w] : bound;
  bool keep[EPT];
  int n = 0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    keep[e] = ord[e] != 0u && ord[e] >= bound;
    n += __popcll(ballot(keep[e]));
  }
  int base = 0;
  if (lane == 0 && n > 0) base = atomicAdd(&L.snsurv, n);
  base = __builtin_amdgcn_readfirstlane(base);
  if (base + n <= kThreads) {
    int off = base;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const uint64_t m = ballot(keep[e]);
      if (keep[e]) L.ssurv[off + lanes_below(m)] = ((uint64_t)ord[e] << 32) |
                                                   (uint64_t)(~(uint32_t)(lo + (int64_t)e * kThreads + tid));
      off += __popcll(m);
    }
  }
  __syncthreads();
  const int ns = L.snsurv;   // the same in every wave
  if (ns <= kThreads) {
    rank_pool<kThreads>(L.ssurv, L.srank, ns, L.sbest);
    if (wave != 0) return;
  } else {
    uint64_t keys[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e)
      keys[e] = ord[e] != 0u
                    ? ((uint64_t)ord[e] << 32) | (uint64_t)(~(uint32_t)(lo + (int64_t)e * kThreads + tid))
                    : 0ull;
    uint64_t* mine16 = L.smerge + wave * 16;
    if (lane < 16) mine16[lane] = 0ull;
    __builtin_amdgcn_wave_barrier();
    const uint64_t t = kth16<EPT>(keys);
    gather_at_least<EPT>(keys, t, mine16);   // the wave's 16 best (fewer if it holds fewer numbers)
    __syncthreads();
    if (wave != 0) return;
    merge_wave_lists<NW>(L.smerge, L.sbest, lane);
  }
  write_chunk_result(L.sbest, splits, k, row, split, out_idx, out_val, part, lane);
}

// One wave per row: merge splits * 16 keys (splits <= 32), each split's 16
// best-first (empty slots 0).  Two lower bounds on the row's 16th best key:
// the largest of the splits' 16th keys (that split holds 16 keys at least
// as large), and the 16th largest among the first ceil(32 / splits) keys of
// every split (16 distinct keys at least as large).  The keys that reach
// both are few (at most 22 per row on the synthetic workloads at 2 to 18
// splits); they are ranked against each other by broadcast LDS compares.
// More than 64 of them (ties at the cut) falls back to the exact 64-bit
// search.
// One wave merges row `row`; sel [16] and ssv [64] are this wave's LDS.
__device__ __forceinline__ void topk_merge_row(const uint64_t* __restrict__ part, int64_t row, int splits, int k,
                                               int32_t* __restrict__ out_idx, float* __restrict__ out_val,
                                               uint64_t* sel_w, uint64_t* ssv_w) {
  constexpr int PER = 8;
  const int lane = lane_id();
  const int n = splits * 16;
  uint64_t keys[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    int s = lane + i * kWave;
    keys[i] = s < n ? part[row * n + s] : 0ull;
  }
  uint64_t b1 = 0ull;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int s = lane + i * kWave;
    if (s < n && (s & 15) == 15 && keys[i] > b1) b1 = keys[i];
  }
  b1 = wave_max_u64(b1);
  // b2: the 16th largest key among the first j keys of every list, with
  // j = ceil(32 / splits) (32 to 62 keys, all in one wave): a subset of the
  // row's keys, so its 16th largest is a lower bound on the row's.  With
  // the lists sorted best-first it lands close to the row's 16th best.
  uint64_t b2 = 0ull;
  {
    const int j = (32 + splits - 1) / splits;
    int nsub = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int s = lane + i * kWave;
      const bool in = s < n && (s & 15) < j;
      const uint64_t m = ballot(in);
      if (in) ssv_w[nsub + lanes_below(m)] = keys[i];
      nsub += __popcll(m);
    }
    __builtin_amdgcn_wave_barrier();
    const uint64_t sk = lane < nsub ? ssv_w[lane] : 0ull;
    int rk = 0;
    for (int l = 0; l < nsub; ++l) rk += ssv_w[l] > sk ? 1 : 0;
    const uint64_t m = ballot(lane < nsub && sk != 0ull && rk == 15);
    if (m) b2 = shfl_u64(sk, __ffsll((unsigned long long)m) - 1);
    __builtin_amdgcn_wave_barrier();
  }
  const uint64_t bound = b1 > b2 ? b1 : b2;
  bool keep[PER];
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    keep[i] = keys[i] != 0ull && keys[i] >= bound;
    cnt += __popcll(ballot(keep[i]));
  }
  uint64_t mine;
  if (cnt <= kWave) {
    if (lane < 16) sel_w[lane] = 0ull;
    int off = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const uint64_t m = ballot(keep[i]);
      if (keep[i]) ssv_w[off + lanes_below(m)] = keys[i];
      off += __popcll(m);
    }
    if (lane >= cnt) ssv_w[lane] = 0ull;   // pad to 64 keys
    __builtin_amdgcn_wave_barrier();
    const uint64_t key = ssv_w[lane];
    const int r = rank_in_lds<kWave>(key, ssv_w);
    if (key != 0ull && r < 16) sel_w[r] = key;
    __builtin_amdgcn_wave_barrier();
    mine = lane < 16 ? sel_w[lane] : 0ull;
  } else {
    const uint64_t t = kth16<PER>(keys);
    const int m = gather_at_least<PER>(keys, t, sel_w);
    __builtin_amdgcn_wave_barrier();
    mine = sorted16(sel_w, m);
  }
  if (lane < k) {
    out_idx[row * k + lane] = (int32_t)key_index(mine);
    out_val[row * k + lane] = key_value(mine);
  }
}

}  // namespace topkd
}  // namespace df2

// select_body.h -- device code of the path selector after the
// projections (select.hip): the in-order sum of split products, the pair
// scores of one (request, position) and the path of one request, as device
// functions that take their block index and LDS from the caller (the
// stand-alone kernels in select.hip, or a persistent kernel).
// Internal; not part of the ABI.
#pragma once

#include "df2_device.h"

namespace df2 {
namespace selectd {


constexpr int kMaxR = 256;
constexpr int kMaxLattice = 63 * 16 * 16;   // T <= 63, K <= 16

// In place: slice 0 of three partial-product buffers (n0, n1, n2 float4 per
// slice, slices k* floats apart) becomes the sum of their `split` slices,
// added in slice order.  One thread per float4; its slices are requested in
// blocks of eight (blocks of sixteen measured slower: 1.2 us per cycle at
// batch 1 / block 8).
__device__ __forceinline__ void slice_reduce_elem(float* __restrict__ p0, int64_t n0, int64_t k0,
                                                  float* __restrict__ p1, int64_t n1, int64_t k1,
                                                  float* __restrict__ p2, int64_t n2, int64_t k2, int split,
                                                  int64_t e) {
  float* p;
  int64_t k;
  if (e < n0) {
    p = p0; k = k0;
  } else if (e < n0 + n1) {
    e -= n0; p = p1; k = k1;
  } else if (e < n0 + n1 + n2) {
    e -= n0 + n1; p = p2; k = k2;
  } else {
    return;
  }
  float* q = p + 4 * e;
  f32x4 acc = *(const f32x4*)q;
  for (int s0 = 1; s0 < split; s0 += 8) {
    f32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = *(const f32x4*)(q + (int64_t)(s0 + u < split ? s0 + u : 0) * k);
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (s0 + u < split) acc += v[u];
  }
  *(f32x4*)q = acc;
}

// TAB = false: ab holds the projected [A | B] row of every candidate
// (B*T*K rows of 2r floats) and a_last the A row of each request's last
// token; H is already summed over its slices.  TAB = true: ab is the
// per-token table [vocab, 2r] and rows are addressed by token id (cand_idx,
// last_tok); ids outside [0, vocab) read zeros, as the projection does for
// them.  H arrives as hsplit slices of partial products (h_k floats apart):
// the first r/4 threads request them before the id-dependent table loads,
// add them in slice order and gate the sum into LDS.
// rows padded to kLd floats: 16-byte aligned, and 16 rows at one column
// fall in 16 different 16-byte bank groups
constexpr int kLd = kMaxR + 4;
template <bool TAB>
struct PairLds {
  __attribute__((aligned(16))) float sG[16 * kLd];            // A(pred) * H_t
  __attribute__((aligned(16))) float sB[16 * kLd];            // B(cand)
  __attribute__((aligned(16))) float sH[TAB ? kMaxR : 4];     // gated H_t (TAB)
  float sP[4][256];                                           // the waves' partial dots
};

// Work-group (256 threads) for row bt = b T + t of the lattices.
template <bool TAB>
__device__ __forceinline__ void pair_epilogue_body(const float* __restrict__ ab, const float* __restrict__ a_last,
                                                   const float* __restrict__ h_part, int gate,
                                                   const float* __restrict__ cand_val,
                                                   const int32_t* __restrict__ cand_idx,
                                                   const int32_t* __restrict__ last_tok, int64_t vocab, int hsplit,
                                                   int64_t h_k, int T, int K, int r, float* __restrict__ scores,
                                                   int bt, PairLds<TAB>& L) {
  float* sG = L.sG;
  float* sB = L.sB;
  float* sH = L.sH;
  auto& sP = L.sP;
  const int b = bt / T, t = bt % T;
  const int tid = threadIdx.x;
  const int npred = t == 0 ? 1 : K;
  const int r4 = r / 4;
  const float* Hp = h_part + (int64_t)bt * r;
  // U_t(b) of this thread's output, requested before the staging loads
  const int oi = tid / 16, oj = tid % 16;
  const float u_j = (oi < K && oj < K) ? cand_val[(int64_t)bt * K + oj] : 0.f;
  // TAB: the first block of H slices (up to 16: all of them), requested
  // before the table loads
  const bool hthr = TAB && tid < r4;
  const float* hp = Hp + 4 * (hthr ? tid : 0);
  f32x4 hv[16];
  if (hthr) {
#pragma unroll
    for (int u = 0; u < 16; ++u) hv[u] = *(const f32x4*)(hp + (int64_t)(u < hsplit ? u : 0) * h_k);
  }
  // each thread stages up to 4 float4 of G and 4 of B (16 rows x 64 float4)
  f32x4 ga[4], gb[4];
  int gi[4], gq[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    int e = tid + u * 256;            // float4 index over [16 rows][r4]
    gi[u] = e / r4;
    gq[u] = e % r4;
    ga[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    gb[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  if (TAB) {
    // every id, then every table row, requested unconditionally (clamped
    // indices; rows that do not count are loaded from row 0 and dropped), so
    // each round has one wait
    const int32_t* pbase = t == 0 ? last_tok + b : cand_idx + (int64_t)(bt - 1) * K;
    const int32_t* cbase = cand_idx + (int64_t)bt * K;
    int32_t pid[4], cid[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int gc = gi[u] < K ? gi[u] : K - 1;
      pid[u] = pbase[t == 0 ? 0 : gc];
      cid[u] = cbase[gc];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool okp = gi[u] < npred && pid[u] >= 0 && pid[u] < vocab;
      const bool okc = gi[u] < K && cid[u] >= 0 && cid[u] < vocab;
      const f32x4 va = *(const f32x4*)(ab + (int64_t)(okp ? pid[u] : 0) * (2 * r) + 4 * gq[u]);
      const f32x4 vb = *(const f32x4*)(ab + (int64_t)(okc ? cid[u] : 0) * (2 * r) + r + 4 * gq[u]);
      if (okp) ga[u] = va;
      if (okc) gb[u] = vb;
    }
  } else {
    // the projection's results, each read once: streaming loads
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (gi[u] < npred) {
        const float* src = t == 0 ? a_last + (int64_t)b * r
                                  : ab + ((int64_t)(bt - 1) * K + gi[u]) * (2 * r);
        ga[u] = __builtin_nontemporal_load((const f32x4*)(src + 4 * gq[u]));
      }
      if (gi[u] < K) gb[u] = __builtin_nontemporal_load((const f32x4*)(ab + ((int64_t)bt * K + gi[u]) * (2 * r) + r + 4 * gq[u]));
    }
  }
  if (TAB) {
    if (hthr) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (u < hsplit) acc += hv[u];
      for (int s0 = 16; s0 < hsplit; s0 += 16) {
#pragma unroll
        for (int u = 0; u < 16; ++u) hv[u] = *(const f32x4*)(hp + (int64_t)(s0 + u < hsplit ? s0 + u : 0) * h_k);
#pragma unroll
        for (int u = 0; u < 16; ++u)
          if (s0 + u < hsplit) acc += hv[u];
      }
      if (gate == 1)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = 1.0f / (1.0f + expf(-acc[e]));
      *(f32x4*)&sH[4 * tid] = acc;
    }
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    if (gi[u] < 16) {
      f32x4 h = f32x4{0.f, 0.f, 0.f, 0.f};
      if (gi[u] < npred) {
        if (TAB) {
          h = *(const f32x4*)&sH[4 * gq[u]];
        } else {
          h = *(const f32x4*)(Hp + 4 * gq[u]);
          if (gate == 1)
#pragma unroll
            for (int e = 0; e < 4; ++e) h[e] = 1.0f / (1.0f + expf(-h[e]));
        }
      }
      *(f32x4*)&sG[gi[u] * kLd + 4 * gq[u]] = ga[u] * h;
      *(f32x4*)&sB[gi[u] * kLd + 4 * gq[u]] = gb[u];
    }
  }
  __syncthreads();
  // Dot products, register-blocked: wave w takes the float4 columns
  // [w r4/4, (w+1) r4/4) of the rows and lane (bi, bj) the 2 x 2 outputs
  // (2bi..2bi+1, 2bj..2bj+1), so every LDS read feeds two products; the
  // waves' partial sums meet in LDS and are added in wave order.
  {
    const int w = tid >> 6, lane = tid & 63;
    const int i0 = 2 * (lane >> 3), j0 = 2 * (lane & 7);
    const int qn = r4 / 4, qa = w * qn;
    const f32x4* g0 = (const f32x4*)&sG[i0 * kLd] + qa;
    const f32x4* g1 = (const f32x4*)&sG[(i0 + 1) * kLd] + qa;
    const f32x4* b0 = (const f32x4*)&sB[j0 * kLd] + qa;
    const f32x4* b1 = (const f32x4*)&sB[(j0 + 1) * kLd] + qa;
    float a00 = 0.f, a01 = 0.f, a10 = 0.f, a11 = 0.f;
    for (int q = 0; q < qn; ++q) {
      const f32x4 x0 = g0[q], x1 = g1[q], y0 = b0[q], y1 = b1[q];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a00 = fmaf(x0[e], y0[e], a00);
        a01 = fmaf(x0[e], y1[e], a01);
        a10 = fmaf(x1[e], y0[e], a10);
        a11 = fmaf(x1[e], y1[e], a11);
      }
    }
    sP[w][i0 * 16 + j0] = a00;
    sP[w][i0 * 16 + j0 + 1] = a01;
    sP[w][(i0 + 1) * 16 + j0] = a10;
    sP[w][(i0 + 1) * 16 + j0 + 1] = a11;
  }
  __syncthreads();
  const int i = oi, j = oj;
  if (i >= K || j >= K) return;
  float* out = scores + ((int64_t)bt * K + i) * K + j;
  if (i >= npred) {
    *out = -INFINITY;
    return;
  }
  const int o = i * 16 + j;
  *out = u_j + (((sP[0][o] + sP[1][o]) + sP[2][o]) + sP[3][o]);
}

// (value, rank) comparison: larger value, then lower rank
__device__ __forceinline__ bool better(float v1, int i1, float v0, int i0) {
  return v1 > v0 || (v1 == v0 && i1 < i0);
}

// Reductions over the 16 lanes of a DPP row (every row reduces its own lanes;
// the caller reads row 0): two quad permutations, then rotations of the row
// by 4 and 8.  The rotations associate sums differently in different lanes,
// so callers take the result of one lane.
template <int C, bool ZF = false>
__device__ __forceinline__ float dppf(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), C, 0xF, 0xF, ZF));
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dppf<0xB1>(v));    // quad_perm [1,0,3,2]
  v = fmaxf(v, dppf<0x4E>(v));    // quad_perm [2,3,0,1]
  v = fmaxf(v, dppf<0x124>(v));   // row_ror:4
  return fmaxf(v, dppf<0x128>(v));   // row_ror:8
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dppf<0xB1>(v);
  v += dppf<0x4E>(v);
  v += dppf<0x124>(v);
  return v + dppf<0x128>(v);
}
// Inclusive prefix sum over the lanes of a row: row_shr by 1, 2, 4, 8 with
// zero fill (the additions of a Hillis-Steele scan in lane order).
__device__ __forceinline__ float row16_prefix(float c) {
  c += dppf<0x111, true>(c);
  c += dppf<0x112, true>(c);
  c += dppf<0x114, true>(c);
  return c + dppf<0x118, true>(c);
}
__device__ __forceinline__ float lane_value(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Keep the better of this lane's (value, rank) and that of the lane the DPP
// control CTRL names (a quad permutation or a row rotation; all lanes
// active).
template <int CTRL>
__device__ __forceinline__ void dpp_better(float& best, int& arg) {
  const float ob = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(best), CTRL, 0xF, 0xF, false));
  const int oa = __builtin_amdgcn_update_dpp(0, arg, CTRL, 0xF, 0xF, false);
  if (better(ob, oa, best, arg)) {
    best = ob;
    arg = oa;
  }
}

// One work-group of four waves per request: all 256 threads stage the
// request's lattice (T*K*K floats) and its candidate ids in LDS with one
// round of loads; the first wave then runs the recursion (the other waves
// compute the same values in step, write nothing and only keep the
// work-group barriers uniform).
constexpr int kPathThreads = 256;
constexpr int kPathLoads = 4;   // 16-byte lattice loads in flight per thread

struct PathLds {
  uint8_t psi[64][16];
  int32_t chosen[64];
  int32_t sIdx[kMaxLattice / 16];
  __attribute__((aligned(16))) float sD[kPathThreads / 64][2][16];
  __attribute__((aligned(16))) float sS[kMaxLattice];
};

// Work-group (kPathThreads threads) for request b.
__device__ __forceinline__ void path_body(const float* __restrict__ scores, const int32_t* __restrict__ cand_idx,
                                          int T, int K, int mode, float inv_tau,
                                          const uint64_t* __restrict__ seed_dev, int b0,
                                          int32_t* __restrict__ path_rank, int32_t* __restrict__ path_tok,
                                          float* __restrict__ q, float* __restrict__ path_score, int b,
                                          PathLds& L) {
  auto& psi = L.psi;
  auto& chosen = L.chosen;
  auto& sIdx = L.sIdx;
  auto& sD = L.sD;
  float* sS = L.sS;
  const int lane = threadIdx.x & 63;
  const bool w0 = threadIdx.x < 64;   // the wave that writes
  {
    const float* g = scores + (int64_t)b * T * K * K;
    const int n = T * K * K;
    const int nk = T * K;
    const int32_t* ci = cand_idx + (int64_t)b * nk;
    // candidate ids (T*K <= 1008: at most four per thread), issued with the
    // lattice loads below
    int32_t cv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = threadIdx.x + u * kPathThreads;
      cv[u] = e < nk ? ci[e] : 0;
    }
    if (((uintptr_t)g & 15) == 0) {
      const f32x4* g4 = (const f32x4*)g;
      const int n4 = n / 4;
      for (int e0 = 0; e0 < n4; e0 += kPathThreads * kPathLoads) {
        f32x4 v[kPathLoads];
#pragma unroll
        for (int u = 0; u < kPathLoads; ++u) {
          const int e = e0 + u * kPathThreads + threadIdx.x;
          v[u] = e < n4 ? g4[e] : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < kPathLoads; ++u) {
          const int e = e0 + u * kPathThreads + threadIdx.x;
          if (e < n4) ((f32x4*)sS)[e] = v[u];
        }
      }
      for (int e = n4 * 4 + threadIdx.x; e < n; e += kPathThreads) sS[e] = g[e];
    } else {
      for (int e = threadIdx.x; e < n; e += kPathThreads) sS[e] = g[e];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = threadIdx.x + u * kPathThreads;
      if (e < nk) sIdx[e] = cv[u];
    }
  }
  __syncthreads();
  const float* S = sS;
  float total = 0.f;

  if (mode == 0) {  // VITERBI
    // lane = 4 j + g: target rank j, predecessors i = 4 g .. 4 g + 3; the
    // four lanes of a quad combine their (value, rank) pairs with two DPP
    // quad permutations.  delta_{t-1} reaches the lanes through a 16-float
    // LDS row of the wave's own (double-buffered by step parity).
    const int jv = lane >> 2, gv = lane & 3, wv = threadIdx.x >> 6;
    if (lane < 16) sD[wv][0][lane] = lane < K ? S[lane] : -INFINITY;
    __builtin_amdgcn_wave_barrier();
    for (int t = 1; t < T; ++t) {
      const float* St = S + (int64_t)t * K * K;
      const f32x4 dp = *(const f32x4*)&sD[wv][(t - 1) & 1][4 * gv];
      float best = -INFINITY;
      int arg = 4 * gv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * gv + e;
        if (i < K && jv < K) {
          const float v = dp[e] + St[i * K + jv];
          if (v > best) {
            best = v;
            arg = i;
          }
        }
      }
      dpp_better<0xB1>(best, arg);   // lane ^ 1
      dpp_better<0x4E>(best, arg);   // lane ^ 2
      if (gv == 0) {
        if (w0) psi[t][jv] = (uint8_t)arg;
        sD[wv][t & 1][jv] = jv < K ? best : -INFINITY;
      }
      __builtin_amdgcn_wave_barrier();
    }
    const float delta = sD[wv][(T - 1) & 1][lane & 15];
    // end argmax over j (lowest rank on ties) across the 16 lanes of row 0:
    // quad permutations, then row rotations (the pair order is total, so
    // every lane of the row ends with the same best pair)
    float bv = (lane < K) ? delta : -INFINITY;
    int bi = lane < K ? lane : 64;
    dpp_better<0xB1>(bv, bi);
    dpp_better<0x4E>(bv, bi);
    dpp_better<0x124>(bv, bi);   // row_ror:4
    dpp_better<0x128>(bv, bi);   // row_ror:8
    __syncthreads();
    if (w0 && lane == 0) {
      int c = bi;
      chosen[T - 1] = c;
      for (int t = T - 1; t >= 1; --t) {
        c = psi[t][c];
        chosen[t - 1] = c;
      }
      total = bv;
    }
    __syncthreads();
  } else {
    const uint64_t seed = (mode == 2) ? seed_dev[0] : 0ull;
    // SAMPLE: position t's uniform depends on (seed, request, t) alone, so
    // lane t draws it before the walk (T <= 63) and each step reads it
    const float ul = (mode == 2 && lane < T) ? cycle_uniform(seed, b0 + b, lane, 0) : 0.f;
    int prev = 0;
    for (int t = 0; t < T; ++t) {
      float v = (lane < K) ? S[((int64_t)t * K + prev) * K + lane] : -INFINITY;
      int pick;
      if (mode == 1) {  // GREEDY
        float bv = v;
        int bi = lane < K ? lane : 64;
        for (int m = 1; m < 64; m <<= 1) {
          float ov = __shfl_xor(bv, m);
          int oi = __shfl_xor(bi, m);
          if (better(ov, oi, bv, bi)) {
            bv = ov;
            bi = oi;
          }
        }
        pick = bi;
        if (w0 && lane < K) q[((int64_t)b * T + t) * K + lane] = lane == pick ? 1.f : 0.f;
      } else {  // SAMPLE
        // max, sum and prefix over the K <= 16 ranks (lanes 0..15, one DPP
        // row); max and sum are taken from lane 0
        const float mx = lane_value(row16_max(v), 0);
        float e = (lane < K) ? expf((v - mx) * inv_tau) : 0.f;
        const float z = lane_value(row16_sum(e), 0);
        float p = e / z;
        // inclusive prefix sum in rank order
        float c = row16_prefix(p);
        const float u = __shfl(ul, t);
        uint64_t over = ballot(lane < K && c > u);
        if (over) {
          pick = __ffsll((unsigned long long)over) - 1;
        } else {  // rounding: take the last rank with mass
          uint64_t nz = ballot(lane < K && p > 0.f);
          pick = nz ? 63 - __clzll((unsigned long long)nz) : 0;
        }
        if (w0 && lane < K) q[((int64_t)b * T + t) * K + lane] = p;
      }
      float sv = lane_value(v, pick);
      total = (t == 0) ? sv : total + sv;
      if (w0 && lane == 0) chosen[t] = pick;
      prev = pick;
    }
    __syncthreads();
  }
  if (!w0) return;
  for (int t = lane; t < T; t += 64) {
    int c = chosen[t];
    path_rank[(int64_t)b * T + t] = c;
    path_tok[(int64_t)b * T + t] = sIdx[t * K + c];
    if (mode == 0)
      for (int k = 0; k < K; ++k) q[((int64_t)b * T + t) * K + k] = k == c ? 1.f : 0.f;
  }
  if (lane == 0 && path_score) path_score[b] = total;
}

}  // namespace selectd
}  // namespace df2

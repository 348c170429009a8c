// verify.hip -- lossless verification of the drafted path against the
// target's logits.
//
// Greedy ("DFlash 2 讓 Qwen3.8-27B 快了兩倍", section "輸出完全一致"; the
// teaikeji explainer, section 五): the emitted tokens are the target's own
// argmax chain -- the accepted drafts, then the target's token at the first
// disagreement (or the bonus token of row T).
// Rejection sampling ("DFlash 2: Keep Drafting Parallel", section "A
// lightweight path selector": rejection sampling restores the exact target
// distribution): accept draft t with probability min(1, p/q); at the first
// rejection draw from max(0, p - q) by index-order inverse CDF.
//
// Both are one streaming pass over the [B, T+1, V] target logits (16-byte
// loads, several work-groups per row, per-row partials merged by a small
// kernel) plus O(B) follow-up work:
//   greedy : row argmax partials -> per-request prefix check;
//   reject : row (argmax, sum of exp) partials -> per request, when the
//            streaming chunks hold at most 16,384 entries: the accept chain,
//            the residual mass of every chunk of the resampled row from the
//            chunk partials, the chunk search and an in-chunk scan, in one
//            work-group; else per (request, vocabulary chunk): the accept
//            chain, then that chunk's residual mass by a pass over it ->
//            chunk search and in-chunk scan.
// Probabilities are fp32, p(v) = 2^((z_v - m) * log2(e) / tau) / s.
#include "verify_body.h"

namespace df2 {
namespace {
using namespace verifyd;

template <int DT>
__global__ __launch_bounds__(kThreads) void argmax_part_kernel(const void* __restrict__ z, int64_t vocab,
                                                               int splits, int64_t chunk,
                                                               uint64_t* __restrict__ part) {
  __shared__ uint64_t sred[kWaves];
  argmax_part_body<DT>(z, vocab, splits, chunk, part, blockIdx.x, sred);
}

__global__ __launch_bounds__(64) void greedy_final_kernel(const uint64_t* __restrict__ part, int splits, int T,
                                                          const int32_t* __restrict__ path_tok,
                                                          int32_t* __restrict__ accept_len,
                                                          int32_t* __restrict__ out_tok) {
  greedy_final_body(part, splits, T, path_tok, accept_len, out_tok, blockIdx.x);
}

// ---------------------------------------------------------------- softmax stats
struct SumExp {
  float c;            // log2(e) / tau
  float m = -INFINITY;
  float s = 0.f;
  int64_t idx = -1;   // lowest index of the running max
  __device__ void one(float x, int64_t i) {
    if (x > m) {
      s = (m == -INFINITY) ? 0.f : s * exp2f((m - x) * c);
      m = x;
      idx = i;
    }
    s += exp2f((x - m) * c);
  }
  template <int N>
  __device__ void group(const float (&x)[N], int64_t i0) {
    float gm = x[0];
#pragma unroll
    for (int e = 1; e < N; ++e) gm = fmaxf(gm, x[e]);
    if (gm > m) {
      s = (m == -INFINITY) ? 0.f : s * exp2f((m - gm) * c);
      m = gm;
#pragma unroll
      for (int e = N - 1; e >= 0; --e)
        if (x[e] == gm) idx = i0 + e;
    }
#pragma unroll
    for (int e = 0; e < N; ++e) s += exp2f((x[e] - m) * c);
  }
  template <int DT>
  __device__ void vec(const u32x4& v, int64_t i0) { vec_as_floats<DT>(*this, v, i0); }
};


template <int DT>
__global__ __launch_bounds__(kThreads) void sumexp_part_kernel(const void* __restrict__ z,
                                                               int64_t vocab, int splits,
                                                               int64_t chunk, float c,
                                                               RowPart* __restrict__ part) {
  __shared__ uint64_t sk[kWaves];
  __shared__ float ss[kWaves];
  const int64_t row = blockIdx.x / splits;
  const int sp = blockIdx.x % splits;
  const int64_t lo = (int64_t)sp * chunk, hi = lo + chunk < vocab ? lo + chunk : vocab;
  const void* rowp = (const char*)z + row * vocab * Elt<DT>::ESZ;
  SumExp f;
  f.c = c;
  stream_row<DT>(rowp, lo, hi, f);
  uint64_t k = f.idx >= 0 ? make_key(f.m, (uint32_t)f.idx) : 0ull;
  float s = f.idx >= 0 ? f.s : 0.f;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    uint64_t k2 = shfl_xor_u64(k, m);
    float s2 = __shfl_xor(s, m);
    // symmetric combine so that both lanes hold the same result
    uint64_t ka = k < k2 ? k : k2, kb = k < k2 ? k2 : k;
    float sa = k < k2 ? s : s2, sb = k < k2 ? s2 : s;
    combine_part(kb, sb, ka, sa, c);
    k = kb;
    s = sb;
  }
  const int wave = threadIdx.x / kWave;
  if (lane_id() == 0) {
    sk[wave] = k;
    ss[wave] = s;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t K0 = sk[0];
    float S0 = ss[0];
    for (int w = 1; w < kWaves; ++w) combine_part(K0, S0, sk[w], ss[w], c);
    RowPart r;
    r.key = K0;
    r.s = S0;
    r.pad = 0.f;
    part[row * splits + sp] = r;
  }
}

// Request b's decision, from one wave (lanes 0 .. 63): row statistics of
// every position (lane t combines the chunk partials of row t), the accept
// chain, the decision record.  With `write` it also stores accept_len, the
// accepted drafts and -1 after the resampled slot (out_tok[n] is left to
// the draw), and the record in dec[b].
template <int DT>
__device__ __forceinline__ DecRec decide_request(const void* __restrict__ z, int64_t vocab,
                                                 const RowPart* __restrict__ part, int splits, int T, int K, float c,
                                                 const int32_t* __restrict__ path_tok,
                                                 const int32_t* __restrict__ path_rank, const float* __restrict__ q,
                                                 uint64_t seed, int b0, int b, bool write,
                                                 int32_t* __restrict__ accept_len, int32_t* __restrict__ out_tok,
                                                 DecRec* __restrict__ dec) {
  const int lane = threadIdx.x & 63;
  // this lane's drafted token and its rank, requested with the row partials
  const int lt = lane < T ? lane : 0;
  const int32_t x = path_tok[(int64_t)b * T + lt];
  const int rk = path_rank[(int64_t)b * T + lt];
  uint64_t k = 0ull;
  float s = 0.f;
  if (lane <= T) {
    const RowPart* p = part + ((int64_t)b * (T + 1) + lane) * splits;
#pragma unroll 8
    for (int i = 0; i < splits; ++i) combine_part(k, s, p[i].key, p[i].s, c);
  }
  // one Philox block per position: its acceptance uniform (word 1) and the
  // draw's uniform should the chain stop there (word 2; the chain then
  // picks lane n's), both off the critical path
  const u64x4 ph = philox4x64_10(seed, 0, (uint64_t)(lane <= T ? lane : 0), (uint64_t)(b0 + b), 0, 0);
  const float u1l = uniform_of_word(ph.w[1]), u2l = uniform_of_word(ph.w[2]);
  bool reject = false;
  if (lane < T) {
    const float qx = (rk >= 0 && rk < K) ? q[((int64_t)b * T + lane) * K + rk] : 0.f;
    float px = 0.f;
    if (x >= 0 && x < vocab) {
      const void* rowp = (const char*)z + ((int64_t)b * (T + 1) + lane) * vocab * Elt<DT>::ESZ;
      float zx = Elt<DT>::one(rowp, x);
      px = exp2f((zx - key_value(k)) * c) / s;
    }
    const bool accept = qx <= 0.f || u1l < px / qx;
    reject = !accept;
  }
  uint64_t rm = ballot(reject);
  const int n = rm ? __ffsll((unsigned long long)rm) - 1 : T;
  uint32_t klo = __shfl((uint32_t)k, n), khi = __shfl((uint32_t)(k >> 32), n);
  float sn = __shfl(s, n);
  uint64_t knn = ((uint64_t)khi << 32) | klo;
  DecRec d;
  d.n = n;
  d.argmax = knn ? (int)key_index(knn) : 0;
  d.m = key_value(knn);
  d.s = sn;
  d.u2 = __shfl(u2l, n);
  d.pad = 0.f;
  if (write) {
    if (lane == 0) {
      accept_len[b] = n;
      dec[b] = d;
    }
    if (lane <= T && lane != n)
      out_tok[(int64_t)b * (T + 1) + lane] = lane < n ? x : -1;
  }
  return d;
}

// residual weight of entry v of the resampled row
struct Residual {
  float m, s, c;
  int ncand;            // candidates falling in the current range
  int32_t cid[16];
  float cq[16];
  __device__ __forceinline__ float w(float x, int64_t v) const {
    float p = exp2f((x - m) * c) / s;
    for (int i = 0; i < ncand; ++i)
      if (cid[i] == v) {
        float r = p - cq[i];
        return r > 0.f ? r : 0.f;
      }
    return p;
  }
};

struct ResidualSum {
  const Residual* R;
  float acc = 0.f;
  __device__ void one(float x, int64_t i) { acc += R->w(x, i); }
  template <int N>
  __device__ void group(const float (&x)[N], int64_t i0) {
#pragma unroll
    for (int e = 0; e < N; ++e) acc += R->w(x[e], i0 + e);
  }
  template <int DT>
  __device__ void vec(const u32x4& v, int64_t i0) { vec_as_floats<DT>(*this, v, i0); }
};

// The resampled row of request b (row n = the first rejected position, or T
// for the bonus draw).
template <int DT>
__device__ __forceinline__ const void* residual_row(const void* z, int64_t vocab, int T, int b, int n) {
  return (const char*)z + ((int64_t)b * (T + 1) + n) * vocab * Elt<DT>::ESZ;
}

// Fill R (wave 0): the row's softmax constants, and the candidates of the
// rejected position that lie in [lo, hi) with their proposal q, in rank
// order; lane k < K fetches candidate k (one round of loads).  The caller
// synchronises the work-group before R is read.
__device__ __forceinline__ void residual_fill(Residual& R, const DecRec& d, int T, int K, float c, int b,
                                              const int32_t* cand_idx, const float* q, int64_t lo,
                                              int64_t hi) {
  if (threadIdx.x >= kWave) return;
  const int lane = threadIdx.x;
  int32_t v = -1;
  float qq = 0.f;
  if (d.n < T && lane < K) {
    v = cand_idx[((int64_t)b * T + d.n) * K + lane];
    qq = q[((int64_t)b * T + d.n) * K + lane];
  }
  const bool in = v >= lo && v < hi;
  const uint64_t m = ballot(in);
  if (in) {
    R.cid[lanes_below(m)] = v;
    R.cq[lanes_below(m)] = qq;
  }
  if (lane == 0) {
    R.m = d.m;
    R.s = d.s;
    R.c = c;
    R.ncand = __popcll(m);
  }
}

// Work-group (b, ch): request b's decision (every work-group of the request
// takes it the same way; chunk 0's stores it and the request's outputs), then
// the residual mass of vocabulary chunk ch of the resampled row.
template <int DT>
__global__ __launch_bounds__(kThreads) void residual_chunk_kernel(
    const void* __restrict__ z, int64_t vocab, const RowPart* __restrict__ part, int splits, int T, int K, float c,
    const int32_t* __restrict__ path_tok, const int32_t* __restrict__ path_rank,
    const int32_t* __restrict__ cand_idx, const float* __restrict__ q, const uint64_t* __restrict__ seed_dev,
    int b0, int rchunks, int64_t rchunk, int32_t* __restrict__ accept_len, int32_t* __restrict__ out_tok,
    DecRec* __restrict__ dec, float* __restrict__ rsum) {
  __shared__ Residual R;
  __shared__ DecRec sd;
  __shared__ float sred[kWaves];
  const int b = blockIdx.x / rchunks, ch = blockIdx.x % rchunks;
  if (threadIdx.x < kWave) {
    const DecRec d = decide_request<DT>(z, vocab, part, splits, T, K, c, path_tok, path_rank, q, seed_dev[0], b0, b,
                                        ch == 0, accept_len, out_tok, dec);
    if (threadIdx.x == 0) sd = d;
  }
  __syncthreads();
  const DecRec d = sd;
  const int64_t lo = (int64_t)ch * rchunk, hi = lo + rchunk < vocab ? lo + rchunk : vocab;
  const void* row = residual_row<DT>(z, vocab, T, b, d.n);
  residual_fill(R, d, T, K, c, b, cand_idx, q, lo, hi);
  __syncthreads();
  ResidualSum f;
  f.R = &R;
  if (lo < hi) stream_row<DT>(row, lo, hi, f);
  float v = wave_sum_f32(f.acc);
  if (lane_id() == 0) sred[threadIdx.x / kWave] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.f;
    for (int w = 0; w < kWaves; ++w) t += sred[w];
    rsum[(int64_t)b * rchunks + ch] = t;
  }
}

constexpr int kFindBlock = 8;   // entries per block of loads in the in-chunk search

// one work-group per request: find the chunk where the running mass passes
// u2 * total, then the entry inside it
template <int DT>
__global__ __launch_bounds__(kThreads) void residual_find_kernel(
    const void* __restrict__ z, int64_t vocab, int T, int K, float c, int rchunks, int64_t rchunk,
    const DecRec* __restrict__ dec, const int32_t* __restrict__ cand_idx,
    const float* __restrict__ q, const float* __restrict__ rsum, int32_t* __restrict__ out_tok) {
  __shared__ Residual R;
  __shared__ float s_target;
  __shared__ int s_chunk;
  __shared__ float swsum[kWaves];
  __shared__ int shit[kWaves], snz[kWaves];
  const int b = blockIdx.x, tid = threadIdx.x;
  const DecRec d = dec[b];
  if (tid < kWave) {  // wave 0: prefix over chunk sums (rchunks <= 64)
    float v = tid < rchunks ? rsum[(int64_t)b * rchunks + tid] : 0.f;
    float incl = v;
    for (int m = 1; m < 64; m <<= 1) {
      float o = __shfl_up(incl, m);
      if (tid >= m) incl += o;
    }
    float total = __shfl(incl, 63);
    float target = d.u2 * total;
    uint64_t over = ballot(tid < rchunks && incl > target);
    uint64_t nz = ballot(tid < rchunks && v > 0.f);
    int ch;
    float before;
    if (!(total > 0.f)) {
      ch = -1;  // no residual mass
      before = 0.f;
    } else if (over) {
      ch = __ffsll((unsigned long long)over) - 1;
      before = __shfl(incl - v, ch);
    } else {
      ch = 63 - __clzll((unsigned long long)nz);
      before = __shfl(incl - v, ch);
    }
    if (tid == 0) {
      s_chunk = ch;
      s_target = target - before;
    }
  }
  __syncthreads();
  const int ch = s_chunk;
  if (ch < 0) {
    if (tid == 0) out_tok[(int64_t)b * (T + 1) + d.n] = d.argmax;
    return;
  }
  const int64_t lo = (int64_t)ch * rchunk, hi = lo + rchunk < vocab ? lo + rchunk : vocab;
  const void* srow = residual_row<DT>(z, vocab, T, b, d.n);
  // contiguous sub-range per thread, in index order; its entries are
  // loaded in blocks of kFindBlock (all loads of a block in flight, clamped
  // to the range); the first block goes out together with the candidate
  // loads, before the barrier, and is kept for the walk below
  const int64_t per = (rchunk + kThreads - 1) / kThreads;
  const int64_t t0 = lo + tid * per, t1 = t0 + per < hi ? t0 + per : hi;
  float x0[kFindBlock];
#pragma unroll
  for (int u = 0; u < kFindBlock; ++u)   // unconditional, clamped into [lo, hi)
    x0[u] = Elt<DT>::one(srow, t0 + u < t1 ? t0 + u : (t1 > t0 ? t1 - 1 : lo));
  residual_fill(R, d, T, K, c, b, cand_idx, q, lo, hi);
  __syncthreads();
  float mine = 0.f;
  for (int64_t v0 = t0; v0 < t1; v0 += kFindBlock) {
    float x[kFindBlock];
#pragma unroll
    for (int u = 0; u < kFindBlock; ++u)
      x[u] = v0 == t0 ? x0[u] : Elt<DT>::one(srow, v0 + u < t1 ? v0 + u : t1 - 1);
#pragma unroll
    for (int u = 0; u < kFindBlock; ++u)
      if (v0 + u < t1) mine += R.w(x[u], v0 + u);
  }
  // prefix over the thread sums: a wave scan, then the earlier waves'
  // totals added in wave order
  const int lane = lane_id(), wave = tid / kWave;
  float incl = mine;
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) {
    const float o = __shfl_up(incl, m);
    if (lane >= m) incl += o;
  }
  float excl = __shfl_up(incl, 1);
  if (lane == 0) excl = 0.f;
  if (lane == kWave - 1) swsum[wave] = incl;
  __syncthreads();
  float pre = 0.f;
  for (int w = 0; w < wave; ++w) pre += swsum[w];
  incl += pre;
  excl += pre;
  // the first thread whose range takes the running sum past the target,
  // else the last thread with residual mass
  const uint64_t over = ballot(incl > s_target), nz = ballot(mine > 0.f);
  if (lane == 0) {
    shit[wave] = over ? wave * kWave + __ffsll((unsigned long long)over) - 1 : kThreads;
    snz[wave] = nz ? wave * kWave + 63 - __clzll((unsigned long long)nz) : -1;
  }
  __syncthreads();
  int hit = kThreads, last_nz = -1;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    hit = shit[w] < hit ? shit[w] : hit;
    last_nz = snz[w] > last_nz ? snz[w] : last_nz;
  }
  const bool found = hit < kThreads;
  const int tsel = found ? hit : last_nz;
  if (tsel < 0) {
    if (tid == 0) out_tok[(int64_t)b * (T + 1) + d.n] = d.argmax;
    return;
  }
  if (tid != tsel) return;
  // the selected thread walks its own range in index order (the first
  // block from the registers loaded above)
  int y = -1;
  float acc = found ? excl : 0.f;
  int64_t lastv = -1;
  for (int64_t v0 = t0; v0 < t1 && y < 0; v0 += kFindBlock) {
    float x[kFindBlock];
#pragma unroll
    for (int u = 0; u < kFindBlock; ++u)
      x[u] = v0 == t0 ? x0[u] : Elt<DT>::one(srow, v0 + u < t1 ? v0 + u : t1 - 1);
#pragma unroll
    for (int u = 0; u < kFindBlock; ++u) {
      const int64_t v = v0 + u;
      if (v < t1 && y < 0) {
        const float wv = R.w(x[u], v);
        if (wv > 0.f) lastv = v;
        acc += wv;
        if (found && acc > s_target) y = (int)v;
      }
    }
  }
  if (y < 0) y = (int)lastv;
  if (y < 0) y = d.argmax;
  out_tok[(int64_t)b * (T + 1) + d.n] = y;
}

// The residual draw in one work-group per request, when the streaming
// pass's chunks hold at most kFuseThreads * kFusePer entries.  The residual
// mass of a chunk needs no second pass over it: off the candidates,
// max(0, p - q) is p, so the chunk's mass is its share of the softmax sum
// (from the chunk's partial of the streaming pass) less min(p, q) of the
// candidates inside it.  Wave 0 takes the decision while the other waves
// fetch every drafted position's candidates, proposals and logits; then the
// chunk masses, the chunk search and one round of loads to scan the chunk.
// Measured at 8 requests, block 8, V = 151,936 (replayed graph): 15.8 us
// against 13.2 + 11.6 us for the two passes above, 77.1 against 87.2 us per
// cycle.  (Looking the candidates up in LDS for every entry, as the
// residual weight above does, took this kernel to 49 us: each lookup is a
// chain of dependent LDS reads.)
constexpr int kFuseThreads = 512;
constexpr int kFuseWaves = kFuseThreads / kWave;
constexpr int kFusePer = 32;   // entries per thread in the in-chunk scan
constexpr int kFuseT = 63;     // drafted positions held in LDS
constexpr int kFuseCand = (kFuseT * 16 + kFuseThreads - kWave - 1) / (kFuseThreads - kWave);

template <int DT>
__global__ __launch_bounds__(kFuseThreads) void residual_fused_kernel(
    const void* __restrict__ z, int64_t vocab, const RowPart* __restrict__ part, int splits, int64_t chunk, int T,
    int K, float c, const int32_t* __restrict__ path_tok, const int32_t* __restrict__ path_rank,
    const int32_t* __restrict__ cand_idx, const float* __restrict__ q, const uint64_t* __restrict__ seed_dev, int b0,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ out_tok, DecRec* __restrict__ dec) {
  using E = Elt<DT>;
  __shared__ Residual R;
  __shared__ DecRec sd;
  __shared__ int32_t scand[kFuseT * 16];
  __shared__ float sq[kFuseT * 16], sz[kFuseT * 16];
  __shared__ float s_target;
  __shared__ int s_chunk;
  __shared__ float swsum[kFuseWaves];
  __shared__ int shit[kFuseWaves], snz[kFuseWaves];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int lane = lane_id(), wave = tid / kWave;
  if (wave == 0) {
    const DecRec d = decide_request<DT>(z, vocab, part, splits, T, K, c, path_tok, path_rank, q, seed_dev[0], b0, b,
                                        true, accept_len, out_tok, dec);
    if (lane == 0) sd = d;
  } else {
    // candidates, proposals and logits of every drafted position (T K <=
    // 1,008 entries over the other waves): ids and q first, then the
    // logits, each round with all its loads in flight
    const int nk = T * K;
    int32_t v[kFuseCand];
    float qq[kFuseCand];
#pragma unroll
    for (int j = 0; j < kFuseCand; ++j) {
      const int e = tid - kWave + j * (kFuseThreads - kWave);
      const int ec = e < nk ? e : 0;
      v[j] = cand_idx[(int64_t)b * nk + ec];
      qq[j] = q[(int64_t)b * nk + ec];
    }
#pragma unroll
    for (int j = 0; j < kFuseCand; ++j) {
      const int e = tid - kWave + j * (kFuseThreads - kWave);
      if (e < nk) {
        const int t = e / K;
        const bool ok = v[j] >= 0 && v[j] < vocab;
        const void* rowp = (const char*)z + ((int64_t)b * (T + 1) + t) * vocab * E::ESZ;
        const float zv = E::one(rowp, ok ? v[j] : 0);
        sz[e] = ok ? zv : -INFINITY;
        scand[e] = ok ? v[j] : -1;
        sq[e] = qq[j];
      }
    }
  }
  __syncthreads();
  const DecRec d = sd;
  const int n = d.n;
  if (wave == 0) {
    // lane k < K: candidate k of row n (its chunk, and min(p, q), the part
    // of p that is not residual; a repeated token counts at its first
    // slot, as in the residual weight), found with shuffles
    const int32_t cv = (n < T && lane < K) ? scand[n * K + lane] : -1;
    const float zc = (n < T && lane < K) ? sz[n * K + lane] : 0.f;
    const float qc = (n < T && lane < K) ? sq[n * K + lane] : 0.f;
    bool dup = false;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int32_t o = __shfl(cv, j);
      dup = dup || (j < lane && o == cv);
    }
    int cch = -1;
    float sub = 0.f;
    if (cv >= 0 && !dup) {
      cch = (int)(cv / chunk);
      const float pk = exp2f((zc - d.m) * c) / d.s;
      sub = pk < qc ? pk : (qc > 0.f ? qc : 0.f);
    }
    // residual mass of chunk `lane` of row n, then the prefix over chunks
    float mass = 0.f;
    if (lane < splits) {
      const RowPart rp = part[((int64_t)b * (T + 1) + n) * splits + lane];
      if (rp.key) mass = exp2f((key_value(rp.key) - d.m) * c) * rp.s / d.s;
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int ck = __shfl(cch, k);
      const float sk = __shfl(sub, k);
      if (ck == lane) mass -= sk;
    }
    mass = (lane < splits && mass > 0.f) ? mass : 0.f;
    float incl = mass;
    for (int m = 1; m < 64; m <<= 1) {
      const float o = __shfl_up(incl, m);
      if (lane >= m) incl += o;
    }
    const float total = __shfl(incl, 63);
    const float target = d.u2 * total;
    const uint64_t over = ballot(lane < splits && incl > target);
    const uint64_t nz = ballot(lane < splits && mass > 0.f);
    int ch;
    float before;
    if (!(total > 0.f)) {
      ch = -1;  // no residual mass
      before = 0.f;
    } else if (over) {
      ch = __ffsll((unsigned long long)over) - 1;
      before = __shfl(incl - mass, ch);
    } else {
      ch = 63 - __clzll((unsigned long long)nz);
      before = __shfl(incl - mass, ch);
    }
    // the chunk's candidates (first slots only), in rank order
    const bool in = cch >= 0 && cch == ch;
    const uint64_t im = ballot(in);
    if (in) {
      R.cid[lanes_below(im)] = cv;
      R.cq[lanes_below(im)] = qc;
    }
    if (lane == 0) {
      R.ncand = __popcll(im);
      s_chunk = ch;
      s_target = target - before;
    }
  }
  __syncthreads();
  const int ch = s_chunk;
  if (ch < 0) {
    if (tid == 0) out_tok[(int64_t)b * (T + 1) + n] = d.argmax;
    return;
  }
  const int64_t lo = (int64_t)ch * chunk, hi = lo + chunk < vocab ? lo + chunk : vocab;
  const void* srow = residual_row<DT>(z, vocab, T, b, n);
  // a contiguous sub-range per thread, in index order, loaded in one round
  // and kept for the walk below: whole 16-byte groups when the chunk starts
  // 16-byte aligned and holds whole groups (every group is then inside
  // [lo, hi)), else single entries clamped into range
  const int64_t len = hi - lo;
  const bool vec = (((uintptr_t)srow + (uintptr_t)lo * E::ESZ) & 15u) == 0 && len % E::VN == 0;
  const int64_t per = vec ? (len + (int64_t)kFuseThreads * E::VN - 1) / ((int64_t)kFuseThreads * E::VN) * E::VN
                          : (len + kFuseThreads - 1) / kFuseThreads;   // <= kFusePer (plan)
  const int64_t t0 = lo + tid * per < hi ? lo + tid * per : hi;
  const int64_t t1 = t0 + per < hi ? t0 + per : hi;
  float x[kFusePer];
  if (vec) {
    constexpr int NV = kFusePer / E::VN;
    const u32x4* vp = (const u32x4*)((const char*)srow + t0 * E::ESZ);
    u32x4 w[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j)
      w[j] = t0 + j * E::VN < t1 ? __builtin_nontemporal_load(vp + j) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < NV; ++j)
#pragma unroll
      for (int e = 0; e < E::VN; ++e) x[j * E::VN + e] = E::vget(w[j], e);
  } else {
#pragma unroll
    for (int u = 0; u < kFusePer; ++u)
      x[u] = u < per ? E::one(srow, t0 + u < t1 ? t0 + u : (t1 > t0 ? t1 - 1 : lo)) : 0.f;
  }
  // weights: p, then max(0, p - q) at the chunk's candidates (held in
  // registers; a thread's range rarely holds one)
  const int nc = R.ncand;
  int32_t rc[16];
  float rq[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    rc[i] = i < nc ? R.cid[i] : -1;
    rq[i] = R.cq[i];
  }
  float wv[kFusePer];
#pragma unroll
  for (int u = 0; u < kFusePer; ++u) wv[u] = t0 + u < t1 ? exp2f((x[u] - d.m) * c) / d.s : 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (rc[i] >= t0 && rc[i] < t1) {
      const int ui = (int)(rc[i] - t0);
#pragma unroll
      for (int u = 0; u < kFusePer; ++u)
        if (u == ui) wv[u] = wv[u] - rq[i] > 0.f ? wv[u] - rq[i] : 0.f;
    }
  }
  float mine = 0.f;
#pragma unroll
  for (int u = 0; u < kFusePer; ++u) mine += wv[u];
  // prefix over the thread sums: a wave scan, then the earlier waves'
  // totals added in wave order
  float incl = mine;
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) {
    const float o = __shfl_up(incl, m);
    if (lane >= m) incl += o;
  }
  float excl = __shfl_up(incl, 1);
  if (lane == 0) excl = 0.f;
  if (lane == kWave - 1) swsum[wave] = incl;
  __syncthreads();
  float pre = 0.f;
  for (int w = 0; w < wave; ++w) pre += swsum[w];
  incl += pre;
  excl += pre;
  // the first thread whose range takes the running sum past the target,
  // else the last thread with residual mass
  const uint64_t over = ballot(incl > s_target), nz = ballot(mine > 0.f);
  if (lane == 0) {
    shit[wave] = over ? wave * kWave + __ffsll((unsigned long long)over) - 1 : kFuseThreads;
    snz[wave] = nz ? wave * kWave + 63 - __clzll((unsigned long long)nz) : -1;
  }
  __syncthreads();
  int hit = kFuseThreads, last_nz = -1;
#pragma unroll
  for (int w = 0; w < kFuseWaves; ++w) {
    hit = shit[w] < hit ? shit[w] : hit;
    last_nz = snz[w] > last_nz ? snz[w] : last_nz;
  }
  const bool found = hit < kFuseThreads;
  const int tsel = found ? hit : last_nz;
  if (tsel < 0) {
    if (tid == 0) out_tok[(int64_t)b * (T + 1) + n] = d.argmax;
    return;
  }
  if (tid != tsel) return;
  // the selected thread walks its own range in index order
  int y = -1;
  float acc = found ? excl : 0.f;
  int64_t lastv = -1;
#pragma unroll
  for (int u = 0; u < kFusePer; ++u) {
    const int64_t vv = t0 + u;
    if (vv < t1 && y < 0) {
      if (wv[u] > 0.f) lastv = vv;
      acc += wv[u];
      if (found && acc > s_target) y = (int)vv;
    }
  }
  if (y < 0) y = (int)lastv;
  if (y < 0) y = d.argmax;
  out_tok[(int64_t)b * (T + 1) + n] = y;
}

}  // namespace

VerifyPlan verify_plan(int B, int T, int64_t vocab) {
  VerifyPlan p;
  const int64_t rows = (int64_t)B * (T + 1);
  // about 1024 work-groups (four per CU): 512 rows take 2 chunks (argmax
  // pass 29.3 against 29.9 us with 4), 256 rows 4 (17.5 against 19.6 with 8)
  int64_t want = (1024 + rows - 1) / (rows > 0 ? rows : 1);
  // a work-group reads 8,192 bf16 entries per pass of its loads (256
  // threads x 4 x 16 bytes); chunks of at most 16,384 entries take two
  const int64_t one_pass = (vocab + 16383) / 16384;
  const int64_t single = (vocab + 8191) / 8192;
  int64_t max_by_size = one_pass;
  // very few rows: smaller chunks (>= 4096 entries) until rows * chunks
  // reaches 256, one work-group per CU (8 rows of 151,936: 32 chunks, 48.8
  // against 51.1 us per cycle with 9; at 64 or more rows 9 chunks stay best)
  const int64_t few = rows > 0 ? 256 / rows : 1;
  if (few > max_by_size) max_by_size = few < vocab / 4096 ? few : vocab / 4096;
  int64_t s = want < max_by_size ? want : max_by_size;
  // rows whose chunks would take three or more passes go to two-pass chunks
  // while that stays within about six work-groups per CU (136 rows: 8 -> 10
  // chunks, 76.5 -> 75.3 us per cycle; 72 rows: 9 -> 10, 88.1 -> 87.6 us)
  if (s > 1 && s < one_pass && rows * one_pass <= 1536) s = one_pass;
  // and into one-pass chunks while that stays within two work-groups per CU
  // (batch 1 / block 16, 16 rows: 16 -> 19 chunks, 48.5 -> 47.7 us per
  // cycle; for every row count up to 6 per CU, batch 8 / block 8 sampled
  // took 74.8 -> 77.0 us with 1,216 work-groups instead of 640)
  if (s < single && rows * single <= 512) s = single;
  if (s < 1) s = 1;
  if (s > 64) s = 64;
  int64_t chunk = (vocab + s - 1) / s;
  chunk = (chunk + 63) / 64 * 64;
  s = (vocab + chunk - 1) / chunk;
  p.splits = (int)s;
  p.chunk = chunk;
  int64_t rc = (vocab + 63) / 64;
  rc = (rc + 2047) / 2048 * 2048;
  if (rc < 4096) rc = 4096;
  p.rchunk = rc;
  p.rchunks = (int)((vocab + rc - 1) / rc);
  // the residual draw in one work-group per request when one round of its
  // loads covers a streaming chunk and the drafted positions fit its LDS
  p.fused = chunk <= (int64_t)kFuseThreads * kFusePer && T <= kFuseT ? 1 : 0;
  size_t off = 0;
  p.off_part = off;
  off += align256((size_t)rows * s * sizeof(RowPart));
  p.off_dec = off;
  off += align256((size_t)B * sizeof(DecRec));
  p.off_rsum = off;
  off += align256((size_t)B * p.rchunks * sizeof(float));
  p.ws_bytes = off;
  return p;
}

hipError_t launch_verify_greedy(const void* z, int dt, int64_t vocab, const int32_t* path_tok,
                                int B, int T, int32_t* accept_len, int32_t* out_tok, void* ws,
                                const VerifyPlan& plan, hipStream_t stream) {
  if (B == 0) return hipSuccess;
  const int64_t rows = (int64_t)B * (T + 1);
  uint64_t* part = (uint64_t*)((char*)ws + plan.off_part);
  dim3 grid((unsigned)(rows * plan.splits)), block(kThreads);
  {
    ProfileScope ps("argmax_part", stream);
    if (dt == 0)
      DF2_TRY(launch(argmax_part_kernel<0>, grid, block, 0, stream, ps, z, vocab, plan.splits, plan.chunk, part));
    else if (dt == 1)
      DF2_TRY(launch(argmax_part_kernel<1>, grid, block, 0, stream, ps, z, vocab, plan.splits, plan.chunk, part));
    else
      DF2_TRY(launch(argmax_part_kernel<2>, grid, block, 0, stream, ps, z, vocab, plan.splits, plan.chunk, part));
  }
  ProfileScope ps("greedy_final", stream);
  DF2_TRY(launch(greedy_final_kernel, dim3(B), dim3(64), 0, stream, ps, part, plan.splits, T, path_tok, accept_len,
                                                         out_tok));
  return hipGetLastError();
}

template <int DT>
static hipError_t reject_launch(const void* z, int64_t vocab, const int32_t* path_tok,
                          const int32_t* path_rank, const int32_t* cand_idx, const float* q, int B,
                          int T, int K, float c, const uint64_t* seed_dev, int b0, int32_t* accept_len,
                          int32_t* out_tok, void* ws, const VerifyPlan& plan, hipStream_t stream) {
  const int64_t rows = (int64_t)B * (T + 1);
  RowPart* part = (RowPart*)((char*)ws + plan.off_part);
  DecRec* dec = (DecRec*)((char*)ws + plan.off_dec);
  float* rsum = (float*)((char*)ws + plan.off_rsum);
  {
    ProfileScope ps("sumexp_part", stream);
    DF2_TRY(launch(sumexp_part_kernel<DT>, dim3((unsigned)(rows * plan.splits)), dim3(kThreads), 0, stream, ps,
        z, vocab, plan.splits, plan.chunk, c, part));
  }
  if (plan.fused) {
    ProfileScope ps("residual_fused", stream);
    DF2_TRY(launch(residual_fused_kernel<DT>, dim3((unsigned)B), dim3(kFuseThreads), 0, stream, ps,
        z, vocab, part, plan.splits, plan.chunk, T, K, c, path_tok, path_rank, cand_idx, q, seed_dev, b0, accept_len,
        out_tok, dec));
    return hipSuccess;
  }
  {
    // the decision (accept chain) is taken inside the residual pass
    ProfileScope ps("residual_chunk", stream);
    DF2_TRY(launch(residual_chunk_kernel<DT>, dim3((unsigned)(B * plan.rchunks)), dim3(kThreads), 0, stream, ps,
        z, vocab, part, plan.splits, T, K, c, path_tok, path_rank, cand_idx, q, seed_dev, b0, plan.rchunks,
        plan.rchunk, accept_len, out_tok, dec, rsum));
  }
  ProfileScope ps("residual_find", stream);
  DF2_TRY(launch(residual_find_kernel<DT>, dim3(B), dim3(kThreads), 0, stream, ps,
      z, vocab, T, K, c, plan.rchunks, plan.rchunk, dec, cand_idx, q, rsum, out_tok));
  return hipSuccess;
}

hipError_t launch_verify_reject(const void* z, int dt, int64_t vocab, const int32_t* path_tok,
                                const int32_t* path_rank, const int32_t* cand_idx, const float* q,
                                int B, int T, int K, float temperature, const uint64_t* seed_dev, int b0,
                                int32_t* accept_len, int32_t* out_tok, void* ws,
                                const VerifyPlan& plan, hipStream_t stream) {
  if (B == 0) return hipSuccess;
  const float c = kLog2e / temperature;
  if (dt == 0)
    return reject_launch<0>(z, vocab, path_tok, path_rank, cand_idx, q, B, T, K, c, seed_dev, b0, accept_len,
                            out_tok, ws, plan, stream);
  if (dt == 1)
    return reject_launch<1>(z, vocab, path_tok, path_rank, cand_idx, q, B, T, K, c, seed_dev, b0, accept_len,
                            out_tok, ws, plan, stream);
  return reject_launch<2>(z, vocab, path_tok, path_rank, cand_idx, q, B, T, K, c, seed_dev, b0, accept_len,
                          out_tok, ws, plan, stream);
}

}  // namespace df2

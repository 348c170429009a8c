// head_reject.hip -- rejection verification straight from the target's last
// hidden states, through its LM head, without writing the logits.
//
// What is computed is the rejection rule of verify.hip ("DFlash 2: Keep
// Drafting Parallel", section "A lightweight path selector": accept draft t
// with probability min(1, p/q), at the first rejection draw from
// max(0, p - q~), else the bonus draw from row T), with the target's logits
// z[b, t, v] = <h[b, t], E_v> (bf16 products, fp32 sums) of the shared LM
// head ("大模型推理，加速王者：DFlash", paragraph before the three-step
// pipeline).  Probabilities are fp32, p(v) = 2^((z_v - m) log2(e) / tau) / s.
//
// Five launches:
//  1. head_stats (lmhead.hip, statistics mode): the logits on the matrix
//     cores in 128 x 128 tiles; per row and 128-token block the online-
//     softmax partial (max key, sum of exp), plus the logits of the row's
//     candidates and drafted token as their blocks go by.
//  2. head_row_reduce: one wave per row folds the row's block partials.
//  3. head_decide: one work-group per request -- the accept chain, the
//     row n that is drawn from, the residual mass of every block of row n
//     (the block's softmax mass minus min(p, q) of the candidates in it),
//     the block where the running mass passes u2 * total, and what is left
//     of u2 * total at its start.
//  4. head_block_logits: the 128 logits of that block of row n, recomputed
//     (a wave per token, fixed-order fp32 dot products).
//  5. head_draw: one wave per request walks the block's residual weights in
//     index order to the drawn token.
// Fallbacks are those of verify.hip: no residual mass -> the row's argmax
// (lowest index); rounding that leaves the running mass short of the target
// -> the last token with positive weight.
#include "df2_device.h"
#include "df2_internal.h"

namespace df2 {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kTokPerGroup = kWaves;                      // block-logit tokens per work-group (a wave each)
constexpr int kGroupsPerBlock = kHeadBlock / kTokPerGroup;

struct HeadDec {   // per-request decision
  int n;           // accepted drafts; the row that is drawn from
  int nb;          // block of the draw; -1: the token is already written
  float target;    // u2 * total minus the mass of the blocks before nb
                   // (+inf: take the block's last token of positive weight)
  float m, s;      // row n's max logit and sum of exp2((z - m) c)
  int argmax;      // row n's argmax (lowest index)
  int pad[2];
};

// one wave per row: the row's block partials folded in index order per
// lane, then across lanes (symmetric: every lane holds the result)
__global__ __launch_bounds__(kThreads) void head_row_reduce_kernel(const BlockStat* __restrict__ stats,
                                                                   int nblocks, int M, float c,
                                                                   BlockStat* __restrict__ rowst) {
  const int row = blockIdx.x * kWaves + wave_id(), lane = lane_id();
  if (row >= M) return;
  const BlockStat* p = stats + (int64_t)row * nblocks;
  uint64_t k = 0ull;
  float s = 0.f;
  // each lane's partials j = lane, lane + 64, ... in index order, requested
  // eight at a time before they are folded
  constexpr int kBatch = 8;
  for (int j0 = lane; j0 < nblocks; j0 += kWave * kBatch) {
    BlockStat v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int j = j0 + u * kWave;
      v[u] = p[j < nblocks ? j : 0];
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (j0 + u * kWave < nblocks) combine_part(k, s, v[u].key, v[u].s, c);
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const uint64_t k2 = shfl_xor_u64(k, m);
    const float s2 = __shfl_xor(s, m);
    uint64_t ka = k < k2 ? k : k2, kb = k < k2 ? k2 : k;
    float sa = k < k2 ? s : s2, sb = k < k2 ? s2 : s;
    combine_part(kb, sb, ka, sa, c);
    k = kb;
    s = sb;
  }
  if (lane == 0) {
    BlockStat r;
    r.key = k;
    r.s = s;
    r.pad = 0.f;
    rowst[row] = r;
  }
}

// residual mass of block j of the drawn row: its softmax mass less
// min(p, q) of the candidates that fall in it (never below zero)
__device__ __forceinline__ float block_mass(const BlockStat& st, int j, float m, float s, float c,
                                            const int32_t* cb, const float* sub) {
  float P = st.key ? exp2f((key_value(st.key) - m) * c) * (st.s / s) : 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i)
    if (cb[i] == j) P -= sub[i];
  return P > 0.f ? P : 0.f;
}

__global__ __launch_bounds__(kThreads) void head_decide_kernel(
    int T, int K, float c, int64_t vocab, int nblocks, const int32_t* __restrict__ path_tok,
    const int32_t* __restrict__ path_rank, const int32_t* __restrict__ cand, const float* __restrict__ q,
    const uint64_t* __restrict__ seed_dev, int b0, const BlockStat* __restrict__ stats,
    const BlockStat* __restrict__ rowst, const float* __restrict__ zc, const float* __restrict__ zx,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ out_tok, HeadDec* __restrict__ dec) {
  __shared__ int s_n, s_arg;
  __shared__ float s_m, s_s, s_u2;
  __shared__ int32_t s_cb[16];
  __shared__ float s_sub[16];
  __shared__ float swsum[kWaves];
  __shared__ int shit[kWaves], snz[kWaves];
  const int b = blockIdx.x, tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int64_t row0 = (int64_t)b * (T + 1);
  if (tid < kWave) {
    const uint64_t seed = seed_dev[0];
    uint64_t k = 0ull;
    float s = 0.f;
    if (lane <= T) {
      const BlockStat r = rowst[row0 + lane];
      k = r.key;
      s = r.s;
    }
    // one Philox block per position: the acceptance uniform (word 1) and
    // the draw's uniform should the chain stop there (word 2)
    const u64x4 ph = philox4x64_10(seed, 0, (uint64_t)(lane <= T ? lane : 0), (uint64_t)(b0 + b), 0, 0);
    const float u2l = uniform_of_word(ph.w[2]);
    bool reject = false;
    int32_t x = -1;
    if (lane < T) {
      x = path_tok[(int64_t)b * T + lane];
      const int rk = path_rank[(int64_t)b * T + lane];
      const float qx = (rk >= 0 && rk < K) ? q[((int64_t)b * T + lane) * K + rk] : 0.f;
      float px = 0.f;
      if (x >= 0 && x < vocab && k) px = exp2f((zx[row0 + lane] - key_value(k)) * c) / s;
      reject = !(qx <= 0.f || uniform_of_word(ph.w[1]) < px / qx);
    }
    const uint64_t rm = ballot(reject);
    const int n = rm ? __ffsll((unsigned long long)rm) - 1 : T;
    const uint64_t kn = shfl_u64(k, n);
    const float sn = __shfl(s, n), mn = key_value(kn);
    const float u2n = __shfl(u2l, n);
    if (lane == 0) {
      s_n = n;
      s_m = mn;
      s_s = sn;
      s_arg = kn ? (int)key_index(kn) : 0;
      s_u2 = u2n;
      accept_len[b] = n;
    }
    if (lane <= T && lane != n) out_tok[row0 + lane] = lane < n ? x : -1;
    // the candidates of a rejected position: their block and min(p, q)
    // (the first of equal candidates only, as the weight of a token takes
    // the first candidate that names it)
    int32_t v = -1;
    float qq = 0.f, sub = 0.f;
    if (n < T && lane < K) {
      v = cand[((int64_t)b * T + n) * K + lane];
      qq = q[((int64_t)b * T + n) * K + lane];
    }
    bool dup = false;
#pragma unroll
    for (int j = 0; j < 16; ++j) {   // every lane takes part in the shuffles
      const int32_t o = __shfl(v, j);
      dup |= j < lane && o == v;
    }
    if (v < 0 || v >= vocab || dup || !kn) {
      v = -1;
    } else {
      const float p = exp2f((zc[(row0 + n) * K + lane] - mn) * c) / sn;
      const float r = p - qq;
      sub = p - (r > 0.f ? r : 0.f);
    }
    if (lane < 16) {
      s_cb[lane] = v >= 0 ? (int)(v / kHeadBlock) : -1;
      s_sub[lane] = sub;
    }
  }
  __syncthreads();
  const int n = s_n;
  const float m = s_m, sn = s_s;
  const BlockStat* st = stats + (row0 + n) * nblocks;
  // contiguous block ranges per thread, in index order
  const int per = (nblocks + kThreads - 1) / kThreads;
  const int j0 = tid * per < nblocks ? tid * per : nblocks;
  const int j1 = j0 + per < nblocks ? j0 + per : nblocks;
  float mine = 0.f;
  for (int j = j0; j < j1; ++j) mine += block_mass(st[j], j, m, sn, c, s_cb, s_sub);
  // prefix over the thread sums (wave scan, then earlier waves in order)
  float incl = mine;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const float u = __shfl_up(incl, o);
    if (lane >= o) incl += u;
  }
  float excl = __shfl_up(incl, 1);
  if (lane == 0) excl = 0.f;
  if (lane == kWave - 1) swsum[wave] = incl;
  __syncthreads();
  float pre = 0.f, total = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    pre += w < wave ? swsum[w] : 0.f;
    total += swsum[w];
  }
  incl += pre;
  excl += pre;
  const float target = s_u2 * total;
  const uint64_t over = ballot(incl > target), nz = ballot(mine > 0.f);
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
  const bool found = hit < kThreads && total > 0.f;
  const int tsel = found ? hit : last_nz;
  if (!(total > 0.f) || tsel < 0) {   // no residual mass: the row's argmax
    if (tid == 0) {
      out_tok[row0 + n] = s_arg;
      HeadDec d{};
      d.n = n;
      d.nb = -1;
      dec[b] = d;
    }
    return;
  }
  if (tid != tsel) return;
  // the selected thread walks its blocks in order
  float acc = found ? excl : 0.f, tin = INFINITY;
  int nbsel = -1, lastj = -1;
  for (int j = j0; j < j1; ++j) {
    const float R = block_mass(st[j], j, m, sn, c, s_cb, s_sub);
    if (R > 0.f) lastj = j;
    if (found && R > 0.f && acc + R > target) {
      nbsel = j;
      tin = target - acc;
      break;
    }
    acc += R;
  }
  if (nbsel < 0) {   // rounding: the block of the last positive mass, its last token
    nbsel = lastj;
    tin = INFINITY;
  }
  HeadDec d{};
  d.n = n;
  d.nb = nbsel;
  d.target = tin;
  d.m = m;
  d.s = sn;
  d.argmax = s_arg;
  if (nbsel < 0) {
    out_tok[row0 + n] = s_arg;
    d.nb = -1;
  }
  dec[b] = d;
}

// the logits of block dec.nb of row (b, n): one wave per token (four per
// work-group, 32 work-groups per request); lane l takes the 16-byte chunks
// l, l + 64, ... of the two rows, all requested before the products, summed
// in chunk order, then a fixed butterfly over the wave
__global__ __launch_bounds__(kThreads) void head_block_logits_kernel(const uint16_t* __restrict__ h,
                                                                     const uint16_t* __restrict__ emb,
                                                                     int64_t vocab, int d, int T,
                                                                     const HeadDec* __restrict__ dec,
                                                                     float* __restrict__ zblk) {
  const int b = blockIdx.x / kGroupsPerBlock, g = blockIdx.x % kGroupsPerBlock;
  const HeadDec dd = dec[b];
  if (dd.nb < 0) return;
  const int tok = g * kTokPerGroup + wave_id(), lane = lane_id();
  const int64_t v = (int64_t)dd.nb * kHeadBlock + tok;
  if (v >= vocab) return;   // the same in the whole wave
  const u32x4* hr = (const u32x4*)(h + ((int64_t)b * (T + 1) + dd.n) * d);
  const u32x4* er = (const u32x4*)(emb + v * d);
  const int nch = d / 8;   // 16-byte chunks per row (d % 64 == 0: a multiple of 8)
  constexpr int kBatch = 8;
  float acc = 0.f;
  for (int c0 = lane; c0 < nch; c0 += kWave * kBatch) {
    u32x4 a[kBatch], e[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int ch = c0 + u * kWave;
      a[u] = hr[ch < nch ? ch : 0];
      e[u] = er[ch < nch ? ch : 0];
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (c0 + u * kWave < nch) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc += bf16_lo(a[u][i]) * bf16_lo(e[u][i]);
          acc += bf16_hi(a[u][i]) * bf16_hi(e[u][i]);
        }
      }
    }
  }
  acc = wave_sum_f32(acc);
  if (lane == 0) zblk[(int64_t)b * kHeadBlock + tok] = acc;
}

// one wave per request: lane L weighs tokens 2 L and 2 L + 1 of the block
// (index order within the lane, then across lanes) and the token where the
// running weight passes the target is the draw
__global__ __launch_bounds__(64) void head_draw_kernel(int T, int K, float c, int64_t vocab,
                                                       const int32_t* __restrict__ cand,
                                                       const float* __restrict__ q,
                                                       const HeadDec* __restrict__ dec,
                                                       const float* __restrict__ zblk,
                                                       int32_t* __restrict__ out_tok) {
  const int b = blockIdx.x, lane = lane_id();
  const HeadDec dd = dec[b];
  if (dd.nb < 0) return;
  int32_t cv = -1;
  float cq = 0.f;
  if (dd.n < T && lane < K) {
    cv = cand[((int64_t)b * T + dd.n) * K + lane];
    cq = q[((int64_t)b * T + dd.n) * K + lane];
  }
  float w[2];
  int64_t v[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    v[e] = (int64_t)dd.nb * kHeadBlock + 2 * lane + e;
    w[e] = 0.f;
    if (v[e] < vocab) w[e] = exp2f((zblk[(int64_t)b * kHeadBlock + 2 * lane + e] - dd.m) * c) / dd.s;
  }
  // the first candidate that names a token sets its weight to max(0, p - q)
  bool hitc[2] = {false, false};
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int32_t o = __shfl(cv, j);
    const float oq = __shfl(cq, j);
#pragma unroll
    for (int e = 0; e < 2; ++e)
      if (!hitc[e] && o >= 0 && o == v[e]) {
        hitc[e] = true;
        const float r = w[e] - oq;
        w[e] = r > 0.f ? r : 0.f;
      }
  }
  const float mine = w[0] + w[1];
  float incl = mine;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const float u = __shfl_up(incl, o);
    if (lane >= o) incl += u;
  }
  float excl = __shfl_up(incl, 1);
  if (lane == 0) excl = 0.f;
  const uint64_t over = ballot(incl > dd.target), nz = ballot(mine > 0.f);
  int sel;
  bool found = over != 0ull;
  if (found) sel = __ffsll((unsigned long long)over) - 1;
  else sel = nz ? 63 - __clzll((unsigned long long)nz) : -1;
  if (lane != (sel < 0 ? 0 : sel)) return;
  int32_t y;
  if (sel < 0) y = dd.argmax;
  else if (found) y = (int32_t)((w[1] > 0.f && !(w[0] > 0.f && excl + w[0] > dd.target)) ? v[1] : v[0]);
  else y = (int32_t)(w[1] > 0.f ? v[1] : v[0]);
  out_tok[(int64_t)b * (T + 1) + dd.n] = y;
}

}  // namespace

HeadRejectPlan head_reject_plan(int B, int T, int64_t vocab, int d, int K) {
  HeadRejectPlan p;
  const int M = B * (T + 1);
  p.lm = lmhead_plan(M, vocab, d, 0);
  size_t off = 0;
  p.off_stats = off;
  off += align256((size_t)M * p.lm.nblocks * sizeof(BlockStat));
  p.off_rowst = off;
  off += align256((size_t)M * sizeof(BlockStat));
  p.off_zc = off;
  off += align256((size_t)M * (K > 0 ? K : 1) * sizeof(float));
  p.off_zx = off;
  off += align256((size_t)M * sizeof(float));
  p.off_dec = off;
  off += align256((size_t)B * sizeof(HeadDec));
  p.off_zblk = off;
  off += align256((size_t)B * kHeadBlock * sizeof(float));
  p.ws_bytes = off;
  return p;
}

hipError_t launch_verify_reject_head(const void* h, const void* emb, int64_t vocab, int d,
                                     const int32_t* path_tok, const int32_t* path_rank, const int32_t* cand_idx,
                                     const float* q, int B, int T, int K, float temperature,
                                     const uint64_t* seed_dev, int b0, int32_t* accept_len, int32_t* out_tok,
                                     void* ws, const HeadRejectPlan& plan, hipStream_t stream) {
  if (B == 0) return hipSuccess;
  const int M = B * (T + 1);
  const float c = kLog2e / temperature;
  char* w = (char*)ws;
  HeadStats hs;
  hs.c = c;
  hs.T = T;
  hs.K = K;
  hs.cand = cand_idx;
  hs.xtok = path_tok;
  hs.stats = (BlockStat*)(w + plan.off_stats);
  hs.zc = (float*)(w + plan.off_zc);
  hs.zx = (float*)(w + plan.off_zx);
  BlockStat* rowst = (BlockStat*)(w + plan.off_rowst);
  HeadDec* dec = (HeadDec*)(w + plan.off_dec);
  float* zblk = (float*)(w + plan.off_zblk);
  DF2_TRY(launch_head_stats(h, emb, vocab, M, d, hs, plan.lm, stream));
  {
    ProfileScope ps("head_row_reduce", stream);
    DF2_TRY(launch(head_row_reduce_kernel, dim3((unsigned)((M + kWaves - 1) / kWaves)), dim3(kThreads), 0, stream,
                   ps, (const BlockStat*)hs.stats, plan.lm.nblocks, M, c, rowst));
  }
  {
    ProfileScope ps("head_decide", stream);
    DF2_TRY(launch(head_decide_kernel, dim3((unsigned)B), dim3(kThreads), 0, stream, ps, T, K, c, vocab,
                   plan.lm.nblocks, path_tok, path_rank, cand_idx, q, seed_dev, b0, (const BlockStat*)hs.stats,
                   (const BlockStat*)rowst, (const float*)hs.zc, (const float*)hs.zx, accept_len, out_tok, dec));
  }
  {
    ProfileScope ps("head_block_logits", stream);
    DF2_TRY(launch(head_block_logits_kernel, dim3((unsigned)(B * kGroupsPerBlock)), dim3(kThreads), 0, stream, ps,
                   (const uint16_t*)h, (const uint16_t*)emb, vocab, d, T, (const HeadDec*)dec, zblk));
  }
  ProfileScope ps("head_draw", stream);
  DF2_TRY(launch(head_draw_kernel, dim3((unsigned)B), dim3(64), 0, stream, ps, T, K, c, vocab, cand_idx, q,
                 (const HeadDec*)dec, (const float*)zblk, out_tok));
  return hipGetLastError();
}

}  // namespace df2

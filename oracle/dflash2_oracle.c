/*
 * dflash2_oracle.c -- plain, slow, obviously correct CPU implementation of the
 * DFlash 2 per-cycle draft-block path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call this code:
 * it is used by the tests, by the smoke check and by the benchmark's
 * CPU-baseline leg, and by nothing else.  It shares no source with the HIP
 * library (no headers, helpers, tables or constants).
 *
 * Sources (the pages; cited by title and section):
 *   [KDP]  "DFlash 2: Keep Drafting Parallel" (Inco AI blog, zh-CN mirror
 *          "DFlash 2：保持并行起草"), sections "The right tokens are already
 *          there", "A lightweight path selector", "A lightweight local
 *          convolution"; Table 1, Table 2, Fig. 1, Fig. 4.
 *   [WC]   "DFlash 2 讓 Qwen3.8-27B 快了兩倍" (wiselychen), section
 *          "DFlash 2 的三個改進" item 2 (pair score, Viterbi) and section
 *          "輸出完全一致" (lossless verification).
 *   [AREX] "Inco AI 发布 DFlash 2" (arex-research), section "85.4% 与 99.5%".
 *   [TEAI] "DFlash2 并行投机解码解读" (teaikeji), sections 二 and 五.
 *
 * Precision: floating-point sums run in double and are rounded once to float
 * at the defined output points.  The path search is defined on float scores
 * with float additions (so that a decision is taken in the precision of the
 * scores it reads); sampling and verification probabilities are double.
 *
 * Parity status of each function is recorded next to it ("pinned by").
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* dtype codes accepted by the oracle (OR_FP64: double logits, accepted by
 * the verification functions only) */
#define OR_FP32 0
#define OR_BF16 1
#define OR_FP16 2
#define OR_FP64 3

/* path modes */
#define OR_PATH_VITERBI 0
#define OR_PATH_GREEDY 1
#define OR_PATH_SAMPLE 2

/* context gate */
#define OR_GATE_IDENTITY 0
#define OR_GATE_SIGMOID 1

/* ------------------------------------------------------------------ */
/* element decoding                                                     */
/* ------------------------------------------------------------------ */

static float bits_to_float(uint32_t u) {
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* bfloat16: the upper 16 bits of an IEEE binary32 */
static float bf16_value(uint16_t b) { return bits_to_float((uint32_t)b << 16); }

/* IEEE binary16 -> float, written out from the format's definition */
static float fp16_value(uint16_t h) {
  int sign = (h >> 15) & 1;
  int expo = (h >> 10) & 0x1f;
  int mant = h & 0x3ff;
  double v;
  if (expo == 0)
    v = ldexp((double)mant, -24); /* subnormal: mant * 2^-14 * 2^-10 */
  else if (expo == 31)
    v = mant ? NAN : INFINITY;
  else
    v = ldexp(1.0 + mant / 1024.0, expo - 15);
  return (float)(sign ? -v : v);
}

static float elem(const void* p, int dt, int64_t i) {
  if (dt == OR_FP32) return ((const float*)p)[i];
  if (dt == OR_BF16) return bf16_value(((const uint16_t*)p)[i]);
  return fp16_value(((const uint16_t*)p)[i]);
}

/* the same in double, with double logits (OR_FP64) read as they are */
static double elemd(const void* p, int dt, int64_t i) {
  if (dt == OR_FP64) return ((const double*)p)[i];
  return (double)elem(p, dt, i);
}

/* ------------------------------------------------------------------ */
/* threads                                                              */
/* ------------------------------------------------------------------ */

void oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int oracle_get_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------ */
/* Philox4x64-10 (Salmon, Moraes, Dror, Shaw: "Parallel Random Numbers: */
/* As Easy as 1, 2, 3", SC'11).  Each round multiplies counter words 0   */
/* and 2 by the two round multipliers, takes the 128-bit products apart  */
/* and mixes the high halves into words 1 and 3 with the round key; the  */
/* key advances by the two Weyl constants between rounds.               */
/* Pinned by: numpy.random.Philox (an independent implementation).      */
/* ------------------------------------------------------------------ */

static void mul_hi_lo_64(uint64_t a, uint64_t b, uint64_t* hi, uint64_t* lo) {
  unsigned __int128 p = (unsigned __int128)a * (unsigned __int128)b;
  *hi = (uint64_t)(p >> 64);
  *lo = (uint64_t)p;
}

void oracle_philox4x64_10(uint64_t key0, uint64_t key1, const uint64_t ctr[4], uint64_t out[4]) {
  const uint64_t mult0 = 0xD2E7470EE14C6C93ULL, mult1 = 0xCA5A826395121157ULL;
  const uint64_t weyl0 = 0x9E3779B97F4A7C15ULL, weyl1 = 0xBB67AE8584CAA73BULL;
  uint64_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
  uint64_t k0 = key0, k1 = key1;
  for (int round = 0; round < 10; ++round) {
    uint64_t hi0, lo0, hi1, lo1;
    mul_hi_lo_64(mult0, x0, &hi0, &lo0);
    mul_hi_lo_64(mult1, x2, &hi1, &lo1);
    uint64_t n0 = hi1 ^ x1 ^ k0;
    uint64_t n1 = lo1;
    uint64_t n2 = hi0 ^ x3 ^ k1;
    uint64_t n3 = lo0;
    x0 = n0; x1 = n1; x2 = n2; x3 = n3;
    k0 += weyl0;
    k1 += weyl1;
  }
  out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

/* A uniform in (0,1) from one 64-bit word: the top 23 bits m give
 * (2m+1) / 2^24, which is exact in binary32 and never 0 or 1. */
double oracle_uniform_from_word(uint64_t w) {
  uint64_t m = w >> 41;
  return (double)(2 * m + 1) * (1.0 / 16777216.0);
}

/* uniform for position t of request b, stream lane 0..3:
 * key = (seed, 0), counter = (t, b, 0, 0). */
static double cycle_uniform(uint64_t seed, int b, int t, int lane) {
  uint64_t ctr[4] = {(uint64_t)t, (uint64_t)b, 0, 0}, out[4];
  oracle_philox4x64_10(seed, 0, ctr, out);
  return oracle_uniform_from_word(out[lane]);
}

/* ------------------------------------------------------------------ */
/* Top-K per row.  [KDP] "The right tokens are already there" and        */
/* "A lightweight path selector": keep the K best candidates of each     */
/* draft position; [AREX] "85.4% 与 99.5%".  Definition: sort the whole  */
/* row by (value descending, index ascending) and keep the first K.      */
/* Values are compared as floats (-0 == +0; equal values -> lower index).*/
/* Pinned by: numpy stable argsort; brute force.                         */
/* ------------------------------------------------------------------ */

typedef struct {
  float v;
  int32_t i;
} vi_pair;

static int by_value_desc_index_asc(const void* pa, const void* pb) {
  const vi_pair* a = (const vi_pair*)pa;
  const vi_pair* b = (const vi_pair*)pb;
  if (a->v > b->v) return -1;
  if (a->v < b->v) return 1;
  return (a->i > b->i) - (a->i < b->i);
}

int oracle_topk(const void* logits, int dt, int64_t rows, int64_t vocab, int k,
                int32_t* out_idx, float* out_val) {
  if (k < 1 || k > vocab) return 3;
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < rows; ++r) {
    vi_pair* row = (vi_pair*)malloc(sizeof(vi_pair) * (size_t)vocab);
    if (!row) { err = 1; continue; }
    for (int64_t v = 0; v < vocab; ++v) {
      row[v].v = elem(logits, dt, r * vocab + v);
      row[v].i = (int32_t)v;
    }
    qsort(row, (size_t)vocab, sizeof(vi_pair), by_value_desc_index_asc);
    for (int j = 0; j < k; ++j) {
      out_idx[r * k + j] = row[j].i;
      out_val[r * k + j] = row[j].v;
    }
    free(row);
  }
  return err ? 1 : 0;
}

/* ------------------------------------------------------------------ */
/* Drafter logits through the LM head shared with the target, then the  */
/* K best per row.  "大模型推理，加速王者：DFlash" (m.163.com), paragraph */
/* before the three-step pipeline: the drafter reuses the target's      */
/* embedding and LM head; [WC] "坑 2"-"坑 4": the selector takes its      */
/* top-k candidates from that dense lm_head.  For each row r (a draft   */
/* position's final hidden state h[r], bf16) and every token v:         */
/*   z[r][v] = sum_k h[r][k] * E[v][k]        (double, E bf16 [V, d])     */
/* then the K best by (z descending, v ascending), as oracle_topk orders */
/* a row.  out_val receives the selected logits in double.               */
/* Pinned by: one-hot embedding rows (each logit is one entry of h,     */
/* known by inspection, down to the last of the d coordinates); a        */
/* permutation of E's rows permutes the indices; scaling h by a power of */
/* two scales the logits exactly; agreement with oracle_topk where the   */
/* logits are exact in float.                                            */
/* ------------------------------------------------------------------ */

typedef struct {
  double v;
  int32_t i;
} dvi_pair;

static int by_dvalue_desc_index_asc(const void* pa, const void* pb) {
  const dvi_pair* a = (const dvi_pair*)pa;
  const dvi_pair* b = (const dvi_pair*)pb;
  if (a->v > b->v) return -1;
  if (a->v < b->v) return 1;
  return (a->i > b->i) - (a->i < b->i);
}

int oracle_lm_head_topk(const uint16_t* h, const uint16_t* emb, int64_t rows, int64_t vocab, int d,
                        int k, int32_t* out_idx, double* out_val) {
  if (k < 1 || k > vocab || d < 1) return 3;
  dvi_pair* z = (dvi_pair*)malloc(sizeof(dvi_pair) * (size_t)vocab);
  double* hr = (double*)malloc(sizeof(double) * (size_t)d);
  if (!z || !hr) {
    free(z);
    free(hr);
    return 1;
  }
  for (int64_t r = 0; r < rows; ++r) {
    for (int q = 0; q < d; ++q) hr[q] = (double)bf16_value(h[r * d + q]);
#pragma omp parallel for schedule(static)
    for (int64_t v = 0; v < vocab; ++v) {
      const uint16_t* e = emb + v * d;
      double acc = 0.0;
      for (int q = 0; q < d; ++q) acc += hr[q] * (double)bf16_value(e[q]);
      z[v].v = acc;
      z[v].i = (int32_t)v;
    }
    qsort(z, (size_t)vocab, sizeof(dvi_pair), by_dvalue_desc_index_asc);
    for (int j = 0; j < k; ++j) {
      out_idx[r * k + j] = z[j].i;
      out_val[r * k + j] = z[j].v;
    }
  }
  free(z);
  free(hr);
  return 0;
}

/* ------------------------------------------------------------------ */
/* Rank-r projections.  [KDP] "A lightweight path selector": A and B     */
/* give each token a compact 256-dimensional embedding and H(h_t) gates  */
/* their match from the position's hidden state.  Reading: A(tok) =     */
/* W_A E[tok], B(tok) = W_B E[tok], H = gate(W_H h_t), W in R^{r x d}.   */
/* out[n][j] = gate(sum_k W[j][k] * x[n][k]) in double.                  */
/* Pinned by: float64 matmul.                                            */
/* ------------------------------------------------------------------ */

static double apply_gate(double z, int gate) {
  if (gate == OR_GATE_SIGMOID) return 1.0 / (1.0 + exp(-z));
  return z;
}

static void project_row(const void* x, int x_dt, int64_t x_off, const uint16_t* w, int d, int r,
                        int gate, double* out) {
  for (int j = 0; j < r; ++j) {
    double acc = 0.0;
    for (int k = 0; k < d; ++k)
      acc += (double)bf16_value(w[(int64_t)j * d + k]) * (double)elem(x, x_dt, x_off + k);
    out[j] = apply_gate(acc, gate);
  }
}

int oracle_project(const void* x, int x_dt, int64_t n, int d, const uint16_t* w, int r, int gate,
                   double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) project_row(x, x_dt, i * d, w, d, r, gate, out + i * r);
  return 0;
}

/* ------------------------------------------------------------------ */
/* Pair scores.  [KDP] "A lightweight path selector", equation          */
/*   S_t(a,b) = U_t(b) + < A(a) (.) H(h_t), B(b) >                      */
/* with U_t(b) the drafter's own logit of candidate b; also [WC] item 2 */
/* (eq. 1).  At t = 0 the only predecessor is the last verified token   */
/* (the traversal starts from it), stored as row a = 0; rows a >= 1 of  */
/* t = 0 are -inf.  For t >= 1 predecessor a ranges over the K          */
/* candidates of position t-1.  Sums in double, rounded once to float.  */
/* Optional outputs: the float-rounded A/B/H (nullable).                */
/* Pinned by: float64 einsum; the H = 0 special case.                   */
/* ------------------------------------------------------------------ */

int oracle_pair_scores(const int32_t* cand_idx, const float* cand_val, const int32_t* last_tok,
                       const void* emb, int emb_dt, int64_t vocab, const uint16_t* h,
                       const uint16_t* w_a, const uint16_t* w_b, const uint16_t* w_h, int B, int T,
                       int K, int d, int r, int gate, float* scores, float* a_last_out,
                       float* a_cand_out, float* b_cand_out, float* h_out) {
  for (int64_t i = 0; i < (int64_t)B * T * K; ++i)
    if (cand_idx[i] < 0 || cand_idx[i] >= vocab) return 3;
  for (int b = 0; b < B; ++b)
    if (last_tok[b] < 0 || last_tok[b] >= vocab) return 3;
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int b = 0; b < B; ++b) {
    double* a_last = (double*)malloc(sizeof(double) * r);
    double* hg = (double*)malloc(sizeof(double) * (size_t)T * r);
    double* ac = (double*)malloc(sizeof(double) * (size_t)T * K * r);
    double* bc = (double*)malloc(sizeof(double) * (size_t)T * K * r);
    if (!a_last || !hg || !ac || !bc) {
      err = 1;
      free(a_last); free(hg); free(ac); free(bc);
      continue;
    }
    project_row(emb, emb_dt, (int64_t)last_tok[b] * d, w_a, d, r, OR_GATE_IDENTITY, a_last);
    for (int t = 0; t < T; ++t) {
      project_row(h, OR_BF16, ((int64_t)b * T + t) * d, w_h, d, r, gate, hg + (size_t)t * r);
      for (int c = 0; c < K; ++c) {
        int64_t tok = cand_idx[((int64_t)b * T + t) * K + c];
        project_row(emb, emb_dt, tok * d, w_a, d, r, OR_GATE_IDENTITY, ac + ((size_t)t * K + c) * r);
        project_row(emb, emb_dt, tok * d, w_b, d, r, OR_GATE_IDENTITY, bc + ((size_t)t * K + c) * r);
      }
    }
    for (int t = 0; t < T; ++t) {
      const double* ht = hg + (size_t)t * r;
      for (int i = 0; i < K; ++i) {
        for (int j = 0; j < K; ++j) {
          int64_t o = (((int64_t)b * T + t) * K + i) * K + j;
          if (t == 0 && i > 0) {
            scores[o] = -INFINITY;
            continue;
          }
          const double* pa = (t == 0) ? a_last : ac + ((size_t)(t - 1) * K + i) * r;
          const double* pb = bc + ((size_t)t * K + j) * r;
          double bigram = 0.0;
          for (int q = 0; q < r; ++q) bigram += pa[q] * ht[q] * pb[q];
          double u = (double)cand_val[((int64_t)b * T + t) * K + j];
          scores[o] = (float)(u + bigram);
        }
      }
    }
    if (a_last_out)
      for (int q = 0; q < r; ++q) a_last_out[(int64_t)b * r + q] = (float)a_last[q];
    if (h_out)
      for (int q = 0; q < T * r; ++q) h_out[(int64_t)b * T * r + q] = (float)hg[q];
    if (a_cand_out)
      for (int q = 0; q < T * K * r; ++q) a_cand_out[(int64_t)b * T * K * r + q] = (float)ac[q];
    if (b_cand_out)
      for (int q = 0; q < T * K * r; ++q) b_cand_out[(int64_t)b * T * K * r + q] = (float)bc[q];
    free(a_last); free(hg); free(ac); free(bc);
  }
  return err ? 1 : 0;
}

/* ------------------------------------------------------------------ */
/* Path through the K x K lattice.                                      */
/*  GREEDY  [KDP] "A lightweight path selector" (start at the last       */
/*          verified token, follow the best successor each step); [AREX].*/
/*  VITERBI [WC] item 2: max-sum dynamic programme over the lattice.     */
/*  SAMPLE  [KDP] same section: sampling draws from the same scores;     */
/*          c_t ~ softmax_j(S_t(c_{t-1}, j) / tau), inverse CDF in rank  */
/*          order with Philox lane 0 at (b, t).                          */
/* Scores and path sums are float with float additions; argmax ties go  */
/* to the lowest candidate rank.  q[b,t,:] is the proposal actually used */
/* (one-hot for the deterministic modes).  margin[b,t] is the relative  */
/* margin of the decision that fixed c_t (see each mode).  b_ids        */
/* (nullable) gives the request index used in the Philox counter of row */
/* b (default b), so that a subset of a batch can be recomputed.        */
/* Pinned by: brute force over all K^T paths; Viterbi >= greedy; the    */
/* rank-independent special case; Monte Carlo for SAMPLE.               */
/* ------------------------------------------------------------------ */

static double rel_margin(double best, double second) {
  if (isinf(second) && second < 0) return INFINITY;
  double den = fabs(best) > 1.0 ? fabs(best) : 1.0;
  return (best - second) / den;
}

static int lowest_argmax(const float* v, int n, int stride, double* margin) {
  int arg = 0;
  float best = v[0];
  for (int j = 1; j < n; ++j)
    if (v[(int64_t)j * stride] > best) {
      best = v[(int64_t)j * stride];
      arg = j;
    }
  if (margin) {
    float second = -INFINITY;
    for (int j = 0; j < n; ++j)
      if (j != arg && v[(int64_t)j * stride] > second) second = v[(int64_t)j * stride];
    *margin = rel_margin(best, second);
  }
  return arg;
}

/* inverse CDF in index order: the smallest index whose running sum
 * exceeds u * total; returns -1 if the running sum never does. */
static int inverse_cdf(const double* w, int n, double u, double total, double* margin) {
  double target = u * total, run = 0.0;
  for (int j = 0; j < n; ++j) {
    double prev = run;
    run += w[j];
    if (run > target) {
      if (margin) {
        double lo = target - prev, hi = run - target;
        *margin = (lo < hi ? lo : hi) / total;
      }
      return j;
    }
  }
  return -1;
}

int oracle_path(const float* scores, const int32_t* cand_idx, int B, int T, int K, int mode,
                double temperature, uint64_t seed, const int32_t* b_ids, int32_t* path_rank,
                int32_t* path_tok, float* q, float* path_score, double* margin) {
  if (mode == OR_PATH_SAMPLE && !(temperature > 0)) return 5;
#pragma omp parallel for schedule(dynamic, 1)
  for (int b = 0; b < B; ++b) {
    const float* S = scores + (int64_t)b * T * K * K;
    int32_t* c = path_rank + (int64_t)b * T;
    double* mg = margin ? margin + (int64_t)b * T : NULL;
    float total = 0.0f;
    if (mode == OR_PATH_VITERBI) {
      float* delta = (float*)malloc(sizeof(float) * (size_t)T * K);
      int* psi = (int*)malloc(sizeof(int) * (size_t)T * K);
      for (int j = 0; j < K; ++j) delta[j] = S[j]; /* t = 0, predecessor row 0 */
      for (int t = 1; t < T; ++t) {
        for (int j = 0; j < K; ++j) {
          float best = -INFINITY;
          int arg = 0;
          for (int i = 0; i < K; ++i) {
            float v = delta[(size_t)(t - 1) * K + i] + S[((int64_t)t * K + i) * K + j];
            if (v > best) {
              best = v;
              arg = i;
            }
          }
          delta[(size_t)t * K + j] = best;
          psi[(size_t)t * K + j] = arg;
        }
      }
      double m_end;
      c[T - 1] = lowest_argmax(delta + (size_t)(T - 1) * K, K, 1, &m_end);
      total = delta[(size_t)(T - 1) * K + c[T - 1]];
      if (mg) mg[T - 1] = m_end;
      for (int t = T - 1; t >= 1; --t) {
        c[t - 1] = psi[(size_t)t * K + c[t]];
        if (mg) {
          float best = -INFINITY, second = -INFINITY;
          for (int i = 0; i < K; ++i) {
            float v = delta[(size_t)(t - 1) * K + i] + S[((int64_t)t * K + i) * K + c[t]];
            if (i == c[t - 1]) best = v;
          }
          for (int i = 0; i < K; ++i) {
            float v = delta[(size_t)(t - 1) * K + i] + S[((int64_t)t * K + i) * K + c[t]];
            if (i != c[t - 1] && v > second) second = v;
          }
          double mm = rel_margin(best, second);
          /* the back-pointer fixes c_{t-1} */
          mg[t - 1] = mm;
        }
      }
      free(delta);
      free(psi);
      for (int t = 0; t < T; ++t)
        for (int j = 0; j < K; ++j) q[((int64_t)b * T + t) * K + j] = (j == c[t]) ? 1.0f : 0.0f;
    } else {
      double* e = (double*)malloc(sizeof(double) * K);
      for (int t = 0; t < T; ++t) {
        int prev = (t == 0) ? 0 : c[t - 1];
        const float* row = S + ((int64_t)t * K + prev) * K;
        int pick;
        if (mode == OR_PATH_GREEDY) {
          double mm;
          pick = lowest_argmax(row, K, 1, &mm);
          if (mg) mg[t] = mm;
          for (int j = 0; j < K; ++j) q[((int64_t)b * T + t) * K + j] = (j == pick) ? 1.0f : 0.0f;
        } else {
          double m = -INFINITY, z = 0.0;
          for (int j = 0; j < K; ++j)
            if ((double)row[j] > m) m = row[j];
          for (int j = 0; j < K; ++j) {
            e[j] = exp(((double)row[j] - m) / temperature);
            z += e[j];
          }
          for (int j = 0; j < K; ++j) e[j] /= z;
          double u0 = cycle_uniform(seed, b_ids ? b_ids[b] : b, t, 0), mm = 0.0;
          pick = inverse_cdf(e, K, u0, 1.0, &mm);
          if (pick < 0) { /* rounding left the running sum below u0 */
            pick = K - 1;
            while (pick > 0 && e[pick] <= 0.0) --pick;
            mm = 0.0;
          }
          if (mg) mg[t] = mm;
          for (int j = 0; j < K; ++j) q[((int64_t)b * T + t) * K + j] = (float)e[j];
        }
        c[t] = pick;
        total = (t == 0) ? row[pick] : total + row[pick];
      }
      free(e);
    }
    for (int t = 0; t < T; ++t) path_tok[(int64_t)b * T + t] = cand_idx[((int64_t)b * T + t) * K + c[t]];
    if (path_score) path_score[b] = total;
  }
  return 0;
}

/* ------------------------------------------------------------------ */
/* Greedy verification.  [WC] "輸出完全一致" and [TEAI] 五: under greedy   */
/* decoding the output equals the target's own token-by-token output.   */
/* y_t = argmax_v Z[b,t,v] (lowest index on ties), t = 0..T; n = the     */
/* longest prefix with path_tok[t] == y_t; emitted = drafts 0..n-1 then  */
/* y_n (the verifier's next token, counted in the acceptance length per  */
/* [KDP] Table 1 caption).  out_tok is -1 after the n+1 emitted tokens.  */
/* Pinned by: the output is the target argmax chain; n <= T; all-agree   */
/* gives n = T and the bonus token.                                      */
/* ------------------------------------------------------------------ */

int oracle_verify_greedy(const void* target, int dt, int64_t vocab, const int32_t* path_tok, int B,
                         int T, int32_t* accept_len, int32_t* out_tok, int32_t* argmax_out) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int b = 0; b < B; ++b) {
    int32_t* y = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T + 1));
    for (int t = 0; t <= T; ++t) {
      int64_t base = ((int64_t)b * (T + 1) + t) * vocab;
      float best = elem(target, dt, base);
      int32_t arg = 0;
      for (int64_t v = 1; v < vocab; ++v) {
        float z = elem(target, dt, base + v);
        if (z > best) {
          best = z;
          arg = (int32_t)v;
        }
      }
      y[t] = arg;
      if (argmax_out) argmax_out[(int64_t)b * (T + 1) + t] = arg;
    }
    int n = 0;
    while (n < T && path_tok[(int64_t)b * T + n] == y[n]) ++n;
    accept_len[b] = n;
    for (int t = 0; t <= T; ++t) {
      int32_t v = -1;
      if (t < n) v = path_tok[(int64_t)b * T + t];
      else if (t == n) v = y[n];
      out_tok[(int64_t)b * (T + 1) + t] = v;
    }
    free(y);
  }
  return 0;
}

/* ------------------------------------------------------------------ */
/* Greedy verification straight from the target's hidden states through  */
/* its LM head: [WC] "輸出完全一致" / [TEAI] 五 (under greedy decoding the  */
/* output is the target's own argmax chain), with the target logits      */
/*   Z[b][t][v] = sum_k h[b][t][k] * E[v][k]   (double; h, E bf16)         */
/* computed here instead of read.  y_t = the lowest v maximising Z[b][t]  */
/* for t = 0..T, then the longest-prefix rule of oracle_verify_greedy.    */
/* margin[b][t] (nullable): Z of the argmax minus the runner-up.          */
/* Pinned by: agreement with oracle_verify_greedy on integer inputs (the */
/* logits are exact in float); one-hot LM-head rows (the argmax is known */
/* by inspection); the output equals the argmax chain.                    */
/* ------------------------------------------------------------------ */

int oracle_verify_greedy_head(const uint16_t* h, const uint16_t* emb, int64_t vocab, int d,
                              const int32_t* path_tok, int B, int T, int32_t* accept_len,
                              int32_t* out_tok, int32_t* argmax_out, double* margin) {
  if (vocab < 1 || d < 1) return 3;
  const int64_t rows = (int64_t)B * (T + 1);
  int32_t* y = (int32_t*)malloc(sizeof(int32_t) * (size_t)rows);
  double* hr = (double*)malloc(sizeof(double) * (size_t)d);
  double* z = (double*)malloc(sizeof(double) * (size_t)vocab);
  if (!y || !hr || !z) {
    free(y); free(hr); free(z);
    return 1;
  }
  for (int64_t r = 0; r < rows; ++r) {
    for (int q = 0; q < d; ++q) hr[q] = (double)bf16_value(h[r * d + q]);
#pragma omp parallel for schedule(static)
    for (int64_t v = 0; v < vocab; ++v) {
      double acc = 0.0;
      for (int q = 0; q < d; ++q) acc += hr[q] * (double)bf16_value(emb[v * d + q]);
      z[v] = acc;
    }
    int64_t arg = 0;
    for (int64_t v = 1; v < vocab; ++v)
      if (z[v] > z[arg]) arg = v;
    double second = -INFINITY;
    for (int64_t v = 0; v < vocab; ++v)
      if (v != arg && z[v] > second) second = z[v];
    y[r] = (int32_t)arg;
    if (argmax_out) argmax_out[r] = (int32_t)arg;
    if (margin) margin[r] = z[arg] - second;
  }
  for (int b = 0; b < B; ++b) {
    const int32_t* yb = y + (int64_t)b * (T + 1);
    int n = 0;
    while (n < T && path_tok[(int64_t)b * T + n] == yb[n]) ++n;
    accept_len[b] = n;
    for (int t = 0; t <= T; ++t) {
      int32_t v = -1;
      if (t < n) v = path_tok[(int64_t)b * T + t];
      else if (t == n) v = yb[n];
      out_tok[(int64_t)b * (T + 1) + t] = v;
    }
  }
  free(y); free(hr); free(z);
  return 0;
}

/* ------------------------------------------------------------------ */
/* Speculative rejection sampling.  [KDP] "A lightweight path selector": */
/* rejection sampling restores the exact target distribution; [WC]       */
/* "輸出完全一致"; [AREX].  With p_t = softmax(Z_t / tau):                */
/*   accept draft t iff u1 < p_t(x_t) / q_t(x_t)   (u1: lane 1 at (b,t)) */
/*   at the first rejection, draw from r(v) = max(0, p_t(v) - q~_t(v)),  */
/*   q~ = q on the candidates and 0 elsewhere, by index-order inverse    */
/*   CDF with u2 (lane 2 at (b,t));                                      */
/*   if all T drafts are accepted, draw the bonus token from p_T with    */
/*   u2 at (b,T).                                                        */
/* All probabilities in double.  A proposal q_t(x_t) <= 0 accepts.  If   */
/* the residual has no mass (rounding only), the lowest argmax of p_t is */
/* emitted and *fallbacks is incremented.                                */
/* b_ids (nullable): request index of row b in the Philox counter.      */
/* margin_accept[b,t]: |u1 - p/q| for each evaluated draft (NaN if not   */
/* evaluated); margin_sample[b]: relative distance of u2 * mass from the */
/* neighbouring CDF steps.                                               */
/* Pinned by: Monte Carlo (the emitted tokens follow p); q = p always    */
/* accepts; tau -> 0 reduces to greedy verification; residual mass       */
/* identity.                                                             */
/* ------------------------------------------------------------------ */

static void softmax_row(const void* target, int dt, int64_t base, int64_t vocab, double tau,
                        double* p) {
  double m = -INFINITY, z = 0.0;
  for (int64_t v = 0; v < vocab; ++v) {
    double x = elemd(target, dt, base + v) / tau;
    if (x > m) m = x;
  }
  for (int64_t v = 0; v < vocab; ++v) {
    p[v] = exp(elemd(target, dt, base + v) / tau - m);
    z += p[v];
  }
  for (int64_t v = 0; v < vocab; ++v) p[v] /= z;
}

int oracle_verify_reject(const void* target, int dt, int64_t vocab, const int32_t* path_tok,
                         const int32_t* path_rank, const int32_t* cand_idx, const float* q, int B,
                         int T, int K, double temperature, uint64_t seed, const int32_t* b_ids,
                         int32_t* accept_len,
                         int32_t* out_tok, double* margin_accept, double* margin_sample,
                         int32_t* fallbacks) {
  if (!(temperature > 0)) return 5;
  int nfb = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : nfb)
  for (int b = 0; b < B; ++b) {
    double* p = (double*)malloc(sizeof(double) * (size_t)vocab);
    double* w = (double*)malloc(sizeof(double) * (size_t)vocab);
    const int bc = b_ids ? b_ids[b] : b; /* request index of the counter */
    int n = T, y = -1;
    if (margin_accept)
      for (int t = 0; t < T; ++t) margin_accept[(int64_t)b * T + t] = NAN;
    for (int t = 0; t < T; ++t) {
      softmax_row(target, dt, ((int64_t)b * (T + 1) + t) * vocab, vocab, temperature, p);
      int32_t x = path_tok[(int64_t)b * T + t];
      double qx = q[((int64_t)b * T + t) * K + path_rank[(int64_t)b * T + t]];
      double u1 = cycle_uniform(seed, bc, t, 1);
      double ratio = qx > 0 ? p[x] / qx : INFINITY;
      if (margin_accept) margin_accept[(int64_t)b * T + t] = fabs(u1 - ratio);
      if (u1 < ratio) continue;
      /* first rejection at t: residual max(0, p - q~) */
      n = t;
      for (int64_t v = 0; v < vocab; ++v) {
        double qv = 0.0;
        for (int k = 0; k < K; ++k)
          if (cand_idx[((int64_t)b * T + t) * K + k] == v) qv = q[((int64_t)b * T + t) * K + k];
        double rv = p[v] - qv;
        w[v] = rv > 0 ? rv : 0.0;
      }
      break;
    }
    if (n == T) {
      softmax_row(target, dt, ((int64_t)b * (T + 1) + T) * vocab, vocab, temperature, p);
      memcpy(w, p, sizeof(double) * (size_t)vocab);
    }
    double mass = 0.0;
    for (int64_t v = 0; v < vocab; ++v) mass += w[v];
    double u2 = cycle_uniform(seed, bc, n, 2), ms = 0.0;
    if (mass > 0) {
      y = inverse_cdf(w, (int)vocab, u2, mass, &ms);
      if (y < 0) { /* rounding left the running sum below u2 * mass */
        y = (int)vocab - 1;
        while (y > 0 && w[y] <= 0.0) --y;
        ms = 0.0;
      }
    } else {
      int64_t arg = 0;
      for (int64_t v = 1; v < vocab; ++v)
        if (p[v] > p[arg]) arg = v;
      y = (int)arg;
      ms = 0.0;
      nfb += 1;
    }
    if (margin_sample) margin_sample[b] = ms;
    accept_len[b] = n;
    for (int t = 0; t <= T; ++t) {
      int32_t v = -1;
      if (t < n) v = path_tok[(int64_t)b * T + t];
      else if (t == n) v = y;
      out_tok[(int64_t)b * (T + 1) + t] = v;
    }
    free(p);
    free(w);
  }
  if (fallbacks) *fallbacks = nfb;
  return 0;
}

/* ------------------------------------------------------------------ */
/* Rejection-sampling verification from the target's hidden states       */
/* through its LM head: the target logits Z[b][t][v] = sum_k h[b][t][k]  */
/* E[v][k] are computed in double (instead of read) and verified as in   */
/* oracle_verify_reject, in double throughout.                           */
/* Pinned by: agreement with oracle_verify_reject on integer inputs,     */
/* whose logits are exact in float (the same uniforms give the same      */
/* accepted lengths and tokens).                                         */
/* ------------------------------------------------------------------ */

int oracle_verify_reject_head(const uint16_t* h, const uint16_t* emb, int64_t vocab, int d,
                              const int32_t* path_tok, const int32_t* path_rank, const int32_t* cand_idx,
                              const float* q, int B, int T, int K, double temperature, uint64_t seed,
                              const int32_t* b_ids, int32_t* accept_len, int32_t* out_tok,
                              double* margin_accept, double* margin_sample, int32_t* fallbacks) {
  if (vocab < 1 || d < 1) return 3;
  const int64_t rows = (int64_t)B * (T + 1);
  double* z = (double*)malloc(sizeof(double) * (size_t)rows * (size_t)vocab);
  double* hr = (double*)malloc(sizeof(double) * (size_t)d);
  if (!z || !hr) {
    free(z); free(hr);
    return 1;
  }
  for (int64_t r = 0; r < rows; ++r) {
    for (int qd = 0; qd < d; ++qd) hr[qd] = (double)bf16_value(h[r * d + qd]);
#pragma omp parallel for schedule(static)
    for (int64_t v = 0; v < vocab; ++v) {
      double acc = 0.0;
      for (int qd = 0; qd < d; ++qd) acc += hr[qd] * (double)bf16_value(emb[v * d + qd]);
      z[r * vocab + v] = acc;
    }
  }
  int rc = oracle_verify_reject(z, OR_FP64, vocab, path_tok, path_rank, cand_idx, q, B, T, K, temperature,
                                seed, b_ids, accept_len, out_tok, margin_accept, margin_sample, fallbacks);
  free(z);
  free(hr);
  return rc;
}

/* ------------------------------------------------------------------ */
/* Two-tap dynamic depthwise convolution.  [KDP] "A lightweight local    */
/* convolution", equation Conv_k(x)_t = k_{t,0} (.) x_t + k_{t,1} (.)     */
/* x_{t-1}; each tap is a learned base kernel plus a small correction    */
/* computed from the current hidden state, one correction per 16         */
/* channels; the first position reads the last verified token's         */
/* representation (Fig. 4).  [WC] item 3; [TEAI] 四.                      */
/* Reading: c = W x_t in R^{2G} (G = d / group), rows 0..G-1 correct the */
/* current tap and rows G..2G-1 the previous tap; channel ch uses group  */
/* ch / group.  x_{-1} = x_prev (zero when absent); base absent = 0.     */
/* y in double, rounded once to float.                                   */
/* Pinned by: identity and shift special cases; group-constant taps;    */
/* linearity in x_{t-1}; brute-force tap recovery.                      */
/* ------------------------------------------------------------------ */

int oracle_dynconv2(const uint16_t* x, const uint16_t* x_prev, const uint16_t* w, const float* base,
                    int B, int L, int d, int group, float* y) {
  if (group < 1 || d % group) return 3;
  int G = d / group;
#pragma omp parallel for collapse(2) schedule(static)
  for (int b = 0; b < B; ++b) {
    for (int t = 0; t < L; ++t) {
      double* c = (double*)malloc(sizeof(double) * 2 * (size_t)G);
      const uint16_t* xt = x + ((int64_t)b * L + t) * d;
      for (int n = 0; n < 2 * G; ++n) {
        double acc = 0.0;
        for (int k = 0; k < d; ++k) acc += (double)bf16_value(w[(int64_t)n * d + k]) * bf16_value(xt[k]);
        c[n] = acc;
      }
      for (int ch = 0; ch < d; ++ch) {
        int g = ch / group;
        double k0 = (base ? (double)base[ch] : 0.0) + c[g];
        double k1 = (base ? (double)base[d + ch] : 0.0) + c[G + g];
        double prev;
        if (t > 0) prev = bf16_value(x[((int64_t)b * L + t - 1) * d + ch]);
        else prev = x_prev ? bf16_value(x_prev[(int64_t)b * d + ch]) : 0.0;
        y[((int64_t)b * L + t) * d + ch] = (float)(k0 * bf16_value(xt[ch]) + k1 * prev);
      }
      free(c);
    }
  }
  return 0;
}

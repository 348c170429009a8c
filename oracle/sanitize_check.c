/*
 * sanitize_check.c -- runs every function of the CPU oracle on small inputs
 * (ragged sizes, K = 1, T = 1, a vocabulary equal to K, NaN-free random
 * values, NULL optional outputs) so that a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer can catch out-of-bounds accesses, leaks and
 * undefined arithmetic in the oracle itself.
 *
 * TEST INFRASTRUCTURE ONLY (built and run by tests/test_oracle_sanitize.py
 * with gcc -fsanitize=address,undefined; never part of the product).
 * Prints "ok" and exits 0 when every call returned 0; a sanitizer finding
 * aborts the process.
 */
#include "dflash2_oracle.c"

#include <stdio.h>

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double urand(void) { /* splitmix64 */
  uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  return (double)(z >> 11) * (1.0 / 9007199254740992.0);
}
static double nrand(void) { return 2.0 * urand() - 1.0; }
static uint16_t to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
static uint16_t* bf16_buf(size_t n, double scale) {
  uint16_t* p = (uint16_t*)malloc(n * sizeof(uint16_t));
  for (size_t i = 0; i < n; ++i) p[i] = to_bf16((float)(scale * nrand()));
  return p;
}
static float* f32_buf(size_t n, double scale) {
  float* p = (float*)malloc(n * sizeof(float));
  for (size_t i = 0; i < n; ++i) p[i] = (float)(scale * nrand());
  return p;
}

#define CHECK(call)                                           \
  do {                                                        \
    int rc_ = (call);                                         \
    if (rc_ != 0) {                                           \
      fprintf(stderr, "%s returned %d\n", #call, rc_);       \
      return 1;                                               \
    }                                                         \
  } while (0)

static int run(int B, int T, int K, int V, int d, int r) {
  const int rows = B * T;
  float* logits = f32_buf((size_t)rows * V, 3.0);
  int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)rows * K);
  float* val = (float*)malloc(sizeof(float) * (size_t)rows * K);
  CHECK(oracle_topk(logits, OR_FP32, rows, V, K, idx, val));
  uint16_t* emb = bf16_buf((size_t)V * d, 0.02);
  uint16_t* h = bf16_buf((size_t)rows * d, 1.0);
  uint16_t* wa = bf16_buf((size_t)r * d, 0.1);
  uint16_t* wb = bf16_buf((size_t)r * d, 0.1);
  uint16_t* wh = bf16_buf((size_t)r * d, 0.01);
  int32_t* last = (int32_t*)malloc(sizeof(int32_t) * B);
  for (int b = 0; b < B; ++b) last[b] = (int32_t)(urand() * V) % V;
  double* proj = (double*)malloc(sizeof(double) * (size_t)rows * r);
  CHECK(oracle_project(h, OR_BF16, rows, d, wh, r, OR_GATE_SIGMOID, proj));
  float* S = (float*)malloc(sizeof(float) * (size_t)rows * K * K);
  float* al = (float*)malloc(sizeof(float) * (size_t)B * r);
  float* ac = (float*)malloc(sizeof(float) * (size_t)rows * K * r);
  float* bc = (float*)malloc(sizeof(float) * (size_t)rows * K * r);
  float* hh = (float*)malloc(sizeof(float) * (size_t)rows * r);
  CHECK(oracle_pair_scores(idx, val, last, emb, OR_BF16, V, h, wa, wb, wh, B, T, K, d, r, OR_GATE_IDENTITY, S,
                           al, ac, bc, hh));
  CHECK(oracle_pair_scores(idx, val, last, emb, OR_BF16, V, h, wa, wb, wh, B, T, K, d, r, OR_GATE_SIGMOID, S,
                           NULL, NULL, NULL, NULL));
  int32_t* prank = (int32_t*)malloc(sizeof(int32_t) * (size_t)rows);
  int32_t* ptok = (int32_t*)malloc(sizeof(int32_t) * (size_t)rows);
  float* q = (float*)malloc(sizeof(float) * (size_t)rows * K);
  float* pscore = (float*)malloc(sizeof(float) * B);
  double* margin = (double*)malloc(sizeof(double) * (size_t)rows);
  int32_t* bids = (int32_t*)malloc(sizeof(int32_t) * B);
  for (int b = 0; b < B; ++b) bids[b] = 100 + b;
  for (int mode = 0; mode < 3; ++mode) {
    CHECK(oracle_path(S, idx, B, T, K, mode, 0.7, 42, NULL, prank, ptok, q, pscore, margin));
    CHECK(oracle_path(S, idx, B, T, K, mode, 1.3, 43, bids, prank, ptok, q, NULL, NULL));
  }
  float* target = f32_buf((size_t)B * (T + 1) * V, 3.0);
  int32_t* acc = (int32_t*)malloc(sizeof(int32_t) * B);
  int32_t* out = (int32_t*)malloc(sizeof(int32_t) * (size_t)B * (T + 1));
  int32_t* am = (int32_t*)malloc(sizeof(int32_t) * (size_t)B * (T + 1));
  CHECK(oracle_verify_greedy(target, OR_FP32, V, ptok, B, T, acc, out, am));
  CHECK(oracle_verify_greedy(target, OR_FP32, V, ptok, B, T, acc, out, NULL));
  double* ma = (double*)malloc(sizeof(double) * (size_t)rows);
  double* ms = (double*)malloc(sizeof(double) * B);
  int32_t fb = 0;
  CHECK(oracle_verify_reject(target, OR_FP32, V, ptok, prank, idx, q, B, T, K, 1.0, 7, NULL, acc, out, ma, ms,
                             &fb));
  CHECK(oracle_verify_reject(target, OR_FP32, V, ptok, prank, idx, q, B, T, K, 0.5, 8, bids, acc, out, NULL,
                             NULL, NULL));
  uint16_t* x = bf16_buf((size_t)B * T * d, 1.0);
  uint16_t* xp = bf16_buf((size_t)B * d, 1.0);
  uint16_t* wc = bf16_buf((size_t)(2 * d / 16) * d, 0.02);
  float* base = f32_buf((size_t)2 * d, 1.0);
  float* y = (float*)malloc(sizeof(float) * (size_t)B * T * d);
  CHECK(oracle_dynconv2(x, xp, wc, base, B, T, d, 16, y));
  CHECK(oracle_dynconv2(x, NULL, wc, NULL, B, T, d, 16, y));
  double* lv = (double*)malloc(sizeof(double) * (size_t)rows * K);
  CHECK(oracle_lm_head_topk(h, emb, rows, V, d, K, idx, lv));
  uint16_t* ht = bf16_buf((size_t)B * (T + 1) * d, 1.0);
  double* mg = (double*)malloc(sizeof(double) * (size_t)B * (T + 1));
  CHECK(oracle_verify_greedy_head(ht, emb, V, d, ptok, B, T, acc, out, am, mg));
  CHECK(oracle_verify_greedy_head(ht, emb, V, d, ptok, B, T, acc, out, NULL, NULL));
  CHECK(oracle_verify_reject_head(ht, emb, V, d, ptok, prank, idx, q, B, T, K, 1.0, 7, bids, acc, out, ma, ms,
                                  &fb));
  CHECK(oracle_verify_reject_head(ht, emb, V, d, ptok, prank, idx, q, B, T, K, 0.6, 8, NULL, acc, out, NULL,
                                  NULL, NULL));
  free(logits); free(idx); free(val); free(emb); free(h); free(wa); free(wb); free(wh); free(last);
  free(proj); free(S); free(al); free(ac); free(bc); free(hh); free(prank); free(ptok); free(q);
  free(pscore); free(margin); free(bids); free(target); free(acc); free(out); free(am); free(ma);
  free(ms); free(x); free(xp); free(wc); free(base); free(y); free(lv); free(ht); free(mg);
  return 0;
}

int main(void) {
  uint64_t ctr[4] = {1, 2, 3, 4}, o[4];
  oracle_philox4x64_10(5, 0, ctr, o);
  if (!(oracle_uniform_from_word(o[0]) > 0.0 && oracle_uniform_from_word(o[0]) < 1.0)) return 1;
  /* B, T, K, V, d, r */
  if (run(1, 3, 4, 1000, 64, 16)) return 1;
  if (run(3, 1, 1, 37, 128, 32)) return 1;
  if (run(2, 5, 16, 16, 64, 16)) return 1;     /* vocabulary equal to K */
  if (run(4, 7, 16, 301, 192, 48)) return 1;
  puts("ok");
  return 0;
}

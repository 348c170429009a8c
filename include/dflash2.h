/*
 * dflash2.h -- C ABI of the DFlash 2 per-cycle draft-block library for
 * AMD Instinct MI355X (gfx950).
 *
 * One decode cycle of DFlash 2 speculative decoding, after the drafter has
 * produced a block of logits:
 *
 *   dflash2_dynconv2       two-tap dynamic depthwise convolution (inside the
 *                          drafter, before/after every attention and MLP
 *                          sublayer)
 *   dflash2_topk           keep the K best candidates of every draft position
 *   dflash2_lm_head_topk   the same from the drafter's hidden states, with
 *                          the shared LM head fused in (logits never stored)
 *   dflash2_pair_scores    score every adjacent candidate pair
 *   dflash2_selector_tables  per-token A/B tables, once per weight set
 *   dflash2_pair_scores_tab  the pair scores with A/B read from those tables
 *                            (or in two halves: dflash2_h_projection, then
 *                            dflash2_pair_scores_tab_from_h)
 *   dflash2_path_viterbi   pick one path through the K x K lattices
 *   dflash2_verify_greedy  accept the longest prefix the target agrees with
 *   dflash2_verify_greedy_head  the same from the target's hidden states,
 *                          with its LM head fused in (logits never stored)
 *   dflash2_verify_reject  speculative rejection sampling with a residual draw
 *   dflash2_verify_reject_head  the same from the target's hidden states,
 *                          with its LM head fused in (logits never stored)
 *   dflash2_cycle_fused    top-K, pair scores, path and greedy verification
 *                          of a small batch in one persistent launch
 *
 * Sources (the pages that define the operations; cited by title/section):
 *   [KDP]  "DFlash 2: Keep Drafting Parallel" (Inco AI blog; zh-CN mirror
 *          "DFlash 2：保持并行起草").
 *   [WC]   "DFlash 2 讓 Qwen3.8-27B 快了兩倍" (wiselychen), section
 *          "DFlash 2 的三個改進" and section "輸出完全一致".
 *   [TEAI] "DFlash2 并行投机解码解读" (teaikeji), sections 二 and 五.
 *   [163]  "大模型推理，加速王者：DFlash" (m.163.com).
 *
 * Conventions for every entry point
 *   - Pointers are DEVICE pointers unless marked "host".  All tensors are
 *     dense, row-major, contiguous.  The caller owns every buffer; the
 *     library never allocates device memory.  Stages that need scratch take
 *     (ws, ws_bytes), sized by the matching *_workspace_bytes() query; the
 *     workspace may be reused between calls that are ordered on one stream.
 *   - Every call is asynchronous on `stream`: it validates its arguments on
 *     the host, enqueues kernels and returns.  It never synchronises, never
 *     allocates and never reads device memory on the host, so it may be
 *     recorded into a HIP graph by stream capture.
 *   - Return value: DF2_OK (0) or a positive df2_status.  Argument errors
 *     are detected before anything is launched; nothing is written then.
 *     A launch failure returns DF2_ERR_HIP.  dflash2_last_error() gives a
 *     thread-local description of the last failure.
 *   - Floating-point inputs named "logits" accept DF2_FP32, DF2_BF16 or
 *     DF2_FP16 (dense heads only, as the selector requires; [WC] deployment
 *     section); any other code returns DF2_ERR_DTYPE.
 *   - Limits: 1 <= K <= 16, K <= vocab, 1 <= T <= 63, vocab < 2^31.
 *   - Results are deterministic: the same inputs (and seed) give the same
 *     bits on every run and every launch geometry.
 */
#ifndef DFLASH2_H
#define DFLASH2_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DF2_OK = 0,
  DF2_ERR_NULL = 1,        /* a required pointer is NULL */
  DF2_ERR_DTYPE = 2,       /* unsupported dtype code */
  DF2_ERR_SHAPE = 3,       /* a size is out of the supported range */
  DF2_ERR_WORKSPACE = 4,   /* ws_bytes smaller than the query returned */
  DF2_ERR_UNSUPPORTED = 5, /* mode / temperature combination not supported */
  DF2_ERR_HIP = 6          /* the HIP runtime reported an error */
} df2_status;

typedef enum { DF2_FP32 = 0, DF2_BF16 = 1, DF2_FP16 = 2 } df2_dtype;

typedef enum { DF2_PATH_VITERBI = 0, DF2_PATH_GREEDY = 1, DF2_PATH_SAMPLE = 2 } df2_path_mode;

typedef enum { DF2_GATE_IDENTITY = 0, DF2_GATE_SIGMOID = 1 } df2_gate;

#define DFLASH2_ABI_VERSION 2

int dflash2_abi_version(void);
/* Static text for a status code (host). */
const char* dflash2_status_string(int status);
/* Thread-local text of the last failure on this thread (host). */
const char* dflash2_last_error(void);
/* Query the current device once and cache its properties; optional (every
 * entry point calls it), but call it before capturing a graph. */
int dflash2_init(void);

/* ------------------------------------------------------------------------
 * Top-K per row.  [KDP] "The right tokens are already there" and "A
 * lightweight path selector": DFlash 2 keeps the K (= 16) best candidates of
 * each draft position instead of only the first.
 *
 *   logits   [rows, vocab] of dtype `dt` (rows = B * T)
 *   out_idx  [rows, k] int32   token ids, best first
 *   out_val  [rows, k] float   their logits (exact: bf16/fp16 -> fp32)
 * Order: value descending; equal values (with -0 == +0) by lower token id.
 * NaN entries are never selected.  ws: see dflash2_topk_workspace_bytes.
 * ------------------------------------------------------------------------ */
size_t dflash2_topk_workspace_bytes(int64_t rows, int64_t vocab, int k);
int dflash2_topk(const void* logits, int dt, int64_t rows, int64_t vocab, int k, int32_t* out_idx,
                 float* out_val, void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Drafter logits through the shared LM head, fused with the top-K, so that
 * the [rows, vocab] logits are never written.  The drafter reuses the
 * target's embedding and LM head ([163] "大模型推理，加速王者：DFlash",
 * paragraph before the three-step pipeline); the selector takes its top-k
 * candidates from that dense head ([WC] 坑 2-4):
 *   z[r, v] = sum_k h[r, k] * emb[v, k]   (bf16 products, fp32 sums)
 *   out_idx / out_val [rows, k]: the k best of each row, as dflash2_topk
 *   orders them (value descending, equal values by lower token id; NaN
 *   never selected); out_val holds the fp32 logits.
 *   h    [rows, d] bf16      final hidden state of each draft position
 *   emb  [vocab, d] bf16     the LM head rows (emb_dt = DF2_BF16)
 * Limits: d % 64 == 0, d <= 65536, 1 <= k <= min(16, vocab).  h and emb
 * 16-byte aligned.  ws: per-token-range best-16 lists, sized by
 * dflash2_lm_head_topk_workspace_bytes (rows x ranges x 16 x 8 bytes; 4 MB
 * at 480 rows).  Deterministic: the same inputs give the same bits.
 * ------------------------------------------------------------------------ */
size_t dflash2_lm_head_topk_workspace_bytes(int rows, int64_t vocab, int d, int k);
int dflash2_lm_head_topk(const void* h, const void* emb, int emb_dt, int64_t vocab, int rows, int d, int k,
                         int32_t* out_idx, float* out_val, void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Pair scores.  [KDP] "A lightweight path selector", equation
 *   S_t(a, b) = U_t(b) + < A(a) (.) H(h_t), B(b) >
 * U_t(b) is the drafter's logit of candidate b (cand_val), A and B give each
 * token a rank-r embedding, H gates the match from the position's hidden
 * state; [WC] eq. 1.  Read as A(tok) = W_A E[tok], B(tok) = W_B E[tok],
 * H_t = gate(W_H h_t) with W in R^{r x d}.  At t = 0 the only predecessor
 * is the last verified token (the traversal starts there).
 *
 *   cand_idx [B, T, K] int32, cand_val [B, T, K] float (from dflash2_topk)
 *   last_tok [B] int32           last verified token of each request
 *   emb      [vocab, d]          token embedding table, dtype emb_dt (BF16)
 *   h        [B, T, d] bf16      drafter hidden state per draft position
 *   w_a, w_b, w_h [r, d] bf16
 *   scores   [B, T, K, K] float  S[b,t,a,b']: a = predecessor rank (t >= 1)
 *            or 0 = last verified token (t = 0; rows a >= 1 of t = 0 are
 *            -inf), b' = candidate rank at t.
 * Limits: d % 64 == 0, 16 <= r <= 256, r % 16 == 0, and the embedding
 * table under 4 GiB (vocab * d * 2 < 2^32; else DF2_ERR_UNSUPPORTED).  Token ids outside
 * [0, vocab) read a zero embedding.  Accumulation: fp32 (MFMA bf16 inputs).
 * ws layout (float, each part 256-byte aligned): AB [B*T*K, 2r] (A in
 * columns 0..r-1, B in r..2r-1), A_last [B, r], H [B*T, r].
 * ------------------------------------------------------------------------ */
size_t dflash2_pair_scores_workspace_bytes(int B, int T, int K, int d, int r);
int dflash2_pair_scores(const int32_t* cand_idx, const float* cand_val, const int32_t* last_tok,
                        const void* emb, int emb_dt, int64_t vocab, const void* h, const void* w_a,
                        const void* w_b, const void* w_h, int B, int T, int K, int d, int r,
                        int gate, float* scores, void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Per-token selector tables.  [KDP] "A lightweight path selector": A and B
 * give every token its own compact rank-r vectors, so they depend on the
 * token alone and can be computed once per weight set:
 *   tab[v] = [ W_A E[v] | W_B E[v] ]      for every v in [0, vocab)
 *   emb  [vocab, d] bf16 (emb_dt = DF2_BF16), w_a, w_b [r, d] bf16
 *   tab  [vocab, 2r] float, caller-owned (vocab * 2r * 4 bytes, 16-byte
 *        aligned): A in columns 0..r-1, B in columns r..2r-1.
 * Same limits and arithmetic as dflash2_pair_scores (fp32 accumulation of
 * bf16 products; the rows equal that call's A and B up to summation order).
 * No workspace.  vocab = 0 is a no-op.
 *
 * dflash2_pair_scores_tab computes the same scores as dflash2_pair_scores
 * with A and B read from such a table: per call only H = gate(W_H h_t) is
 * projected (ws: dflash2_pair_scores_tab_workspace_bytes, H's partial
 * products over d).  cand_idx, cand_val, last_tok, h, w_h, scores, gate
 * and the limits are those of dflash2_pair_scores; tab [vocab, 2r] float as
 * above.  Token ids outside [0, vocab) read zero A and B rows.
 *
 * The same call in two halves, so that H (which depends on the drafter's
 * hidden states alone, not on the candidates) can run on another stream
 * while the candidates are selected: dflash2_h_projection writes H's
 * partial products into ws (same size), and dflash2_pair_scores_tab_from_h
 * reads them from ws to finish the scores.  The caller orders the two
 * (same stream, or an event) and passes the same B, T, d, r to both;
 * ws must not be reused in between.
 * ------------------------------------------------------------------------ */
int dflash2_selector_tables(const void* emb, int emb_dt, int64_t vocab, int d, const void* w_a,
                            const void* w_b, int r, float* tab, hipStream_t stream);
size_t dflash2_pair_scores_tab_workspace_bytes(int B, int T, int d, int r);
int dflash2_h_projection(const void* h, const void* w_h, int B, int T, int d, int r, void* ws, size_t ws_bytes,
                         hipStream_t stream);
int dflash2_pair_scores_tab_from_h(const int32_t* cand_idx, const float* cand_val, const int32_t* last_tok,
                                   const float* tab, int64_t vocab, int B, int T, int K, int d, int r, int gate,
                                   float* scores, const void* ws, size_t ws_bytes, hipStream_t stream);
int dflash2_pair_scores_tab(const int32_t* cand_idx, const float* cand_val, const int32_t* last_tok,
                            const float* tab, int64_t vocab, const void* h, const void* w_h, int B, int T,
                            int K, int d, int r, int gate, float* scores, void* ws, size_t ws_bytes,
                            hipStream_t stream);

/* ------------------------------------------------------------------------
 * Path through the lattice.
 *   DF2_PATH_GREEDY  [KDP] "A lightweight path selector": from the last
 *                    verified token follow the best successor at each step.
 *   DF2_PATH_VITERBI [WC] "DFlash 2 的三個改進" item 2: max-sum dynamic
 *                    programme over the lattice.
 *   DF2_PATH_SAMPLE  [KDP] same section: the sampled path draws from the
 *                    same scores; c_t ~ softmax_j(S_t(c_{t-1}, j) / tau),
 *                    inverse CDF in candidate-rank order with Philox4x64-10
 *                    key (seed, 0), counter (t, b0 + b, 0, 0), word 0.
 * Path sums are float additions; argmax ties go to the lowest rank.
 *
 *   scores     [B, T, K, K] float     cand_idx [B, T, K] int32
 *   seed_dev   [1] uint64 (device; read by SAMPLE only, may be NULL else)
 *   b0         index of this call's first request in the batch the seed
 *              covers: request b of the call draws the counter of request
 *              b0 + b, so a batch split over several calls draws the same
 *              uniforms as one call over the whole batch (0 <= b0,
 *              b0 + B < 2^31; else DF2_ERR_SHAPE)
 *   path_rank  [B, T] int32  chosen candidate rank per position
 *   path_tok   [B, T] int32  chosen token id
 *   q          [B, T, K] float  the proposal the step drew from (one-hot for
 *              VITERBI / GREEDY), for dflash2_verify_reject
 *   path_score [B] float (nullable)  float sum of S along the path
 * SAMPLE needs temperature > 0 (else DF2_ERR_UNSUPPORTED).
 * ------------------------------------------------------------------------ */
int dflash2_path_viterbi(const float* scores, const int32_t* cand_idx, int B, int T, int K, int mode,
                         float temperature, const uint64_t* seed_dev, int b0, int32_t* path_rank,
                         int32_t* path_tok, float* q, float* path_score, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Two-tap dynamic depthwise convolution.  [KDP] "A lightweight local
 * convolution", equation Conv_k(x)_t = k_{t,0} (.) x_t + k_{t,1} (.) x_{t-1};
 * each tap is a learned base kernel plus a correction computed from the
 * current hidden state, one correction per `group` (= 16) channels; the first
 * position reads the last verified token (Fig. 4).
 * Reading: c_t = W x_t in R^{2G}, G = d / group; channel ch uses
 *   k0 = base[0][ch] + c_t[ch / group],  k1 = base[1][ch] + c_t[G + ch / group].
 *
 *   x      [B, L, d] bf16         x_prev [B, d] bf16 (nullable -> zeros)
 *   w      [2G, d] bf16           base   [2, d] float (nullable -> zeros)
 *   y      [B, L, d] of y_dt (DF2_BF16, round to nearest even, or DF2_FP32)
 * Limits: group == 16, d % 64 == 0, 1 <= L.  Accumulation fp32.  y must not
 * overlap x or x_prev.  ws: see dflash2_dynconv2_workspace_bytes.
 * ------------------------------------------------------------------------ */
size_t dflash2_dynconv2_workspace_bytes(int B, int L, int d, int group);
int dflash2_dynconv2(const void* x, const void* x_prev, const void* w, const float* base, int B,
                     int L, int d, int group, void* y, int y_dt, void* ws, size_t ws_bytes,
                     hipStream_t stream);

/* ------------------------------------------------------------------------
 * Greedy verification.  [WC] "輸出完全一致", [TEAI] 五: under greedy
 * decoding the output is the target's own token-by-token output.
 * y_t = argmax_v Z[b,t,v] (lowest id on ties) for t = 0..T; n = longest
 * prefix with path_tok[b,t] == y_t; emitted: path_tok[b,0..n-1] then y_n.
 *
 *   target_logits [B, T+1, vocab] of dtype dt (row T gives the bonus token)
 *   path_tok      [B, T] int32
 *   accept_len    [B] int32     n (0..T); acceptance length = n + 1
 *   out_tok       [B, T+1] int32 the n+1 emitted tokens, then -1
 * ------------------------------------------------------------------------ */
size_t dflash2_verify_workspace_bytes(int B, int T, int64_t vocab);
int dflash2_verify_greedy(const void* target_logits, int dt, int64_t vocab, const int32_t* path_tok,
                          int B, int T, int32_t* accept_len, int32_t* out_tok, void* ws,
                          size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Greedy verification that allocates nothing, for callers that cannot
 * allocate device memory or hand over a workspace (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation).
 * Same arguments, results and errors as dflash2_verify_greedy, without
 * (ws, ws_bytes): its scratch is a fixed device array of
 * dflash2_verify_greedy_noalloc_max_bytes() bytes (1 MiB), one per GPU,
 * held until the process ends.  A size whose
 * dflash2_verify_workspace_bytes(B, T, vocab) exceeds that returns
 * DF2_ERR_WORKSPACE before anything is launched (batch 64 x block 16 at
 * vocab 262,144 needs 34 KB; up to about 2,300 requests of block 16 fit).  The array's address is looked up once per
 * device, by dflash2_init or by the first call on that device; call
 * dflash2_init on each device before capturing a graph.  Every call on a
 * GPU shares that GPU's array: calls that may overlap on one GPU (other
 * streams, other threads) race and must be ordered by the caller.  Nothing
 * in the array needs to start at zero; it keeps the last call's contents.
 * ------------------------------------------------------------------------ */
size_t dflash2_verify_greedy_noalloc_max_bytes(void);
int dflash2_verify_greedy_noalloc(const void* target_logits, int dt, int64_t vocab, const int32_t* path_tok,
                                  int B, int T, int32_t* accept_len, int32_t* out_tok, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Greedy verification with the target's LM head fused in: the target
 * logits are computed from the target's final hidden states and argmaxed
 * on the fly, never stored ([WC] "輸出完全一致", [TEAI] 五: under greedy
 * decoding the output is the target's own token-by-token argmax chain):
 *   Z[b, t, v] = sum_k h[b, t, k] * emb[v, k]  (bf16 products, fp32 sums)
 *   y_t = argmax_v Z[b, t, v] (lowest id on ties), then the rule of
 *   dflash2_verify_greedy: n = longest prefix with path_tok == y,
 *   out_tok = (path_tok[0..n-1], y_n, -1 ...).
 *   h    [B, T+1, d] bf16  the target's final hidden state at each
 *                          verified position (row T gives the bonus token)
 *   emb  [vocab, d] bf16   the target's LM head rows (emb_dt = DF2_BF16)
 *   path_tok [B, T]; accept_len [B]; out_tok [B, T+1] as in
 *   dflash2_verify_greedy.
 * Limits: d % 64 == 0, d <= 65536, 1 <= T <= 63, B <= 16384.
 * ws: per-token-range argmax keys, dflash2_verify_greedy_head_workspace_bytes.
 * ------------------------------------------------------------------------ */
size_t dflash2_verify_greedy_head_workspace_bytes(int B, int T, int64_t vocab, int d);
int dflash2_verify_greedy_head(const void* h, const void* emb, int emb_dt, int64_t vocab, int d,
                               const int32_t* path_tok, int B, int T, int32_t* accept_len, int32_t* out_tok,
                               void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Speculative rejection sampling.  [KDP] "A lightweight path selector":
 * rejection sampling restores the exact target distribution; [WC]
 * "輸出完全一致".  With p_t = softmax(Z_t / tau):
 *   accept draft t iff u1 < p_t(x_t) / q_t(x_t)        (word 1 at (t, b0+b))
 *   at the first rejection draw from max(0, p_t - q~_t) (q~ = q on the
 *   candidates of position t, 0 elsewhere) by index-order inverse CDF with
 *   u2 (word 2 at (t, b0+b)); if every draft is accepted, draw the bonus
 *   token from p_T with word 2 at (T, b0+b).
 * Uniforms: Philox4x64-10, key (seed, 0), counter (t, b0 + b, 0, 0); a
 * word w maps to (2 * (w >> 41) + 1) * 2^-24.  q_t(x_t) <= 0 accepts.
 *
 *   target_logits [B, T+1, vocab]; path_tok, path_rank [B, T] int32;
 *   cand_idx [B, T, K] int32; q [B, T, K] float (from dflash2_path_viterbi)
 *   seed_dev [1] uint64 (device)
 *   b0       index of this call's first request in the batch the seed
 *            covers (as in dflash2_path_viterbi): a sub-range of a batch
 *            (pointers offset by b0 requests, B requests) draws the same
 *            uniforms as the whole batch in one call
 *   accept_len [B], out_tok [B, T+1] as in dflash2_verify_greedy
 * Needs temperature > 0 (else DF2_ERR_UNSUPPORTED).  Probabilities fp32.
 * ------------------------------------------------------------------------ */
int dflash2_verify_reject(const void* target_logits, int dt, int64_t vocab, const int32_t* path_tok,
                          const int32_t* path_rank, const int32_t* cand_idx, const float* q, int B,
                          int T, int K, float temperature, const uint64_t* seed_dev, int b0,
                          int32_t* accept_len, int32_t* out_tok, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/* ------------------------------------------------------------------------
 * Rejection sampling with the target's LM head fused in: the rule of
 * dflash2_verify_reject ([KDP] "A lightweight path selector"; [WC]
 * "輸出完全一致") on the logits
 *   Z[b, t, v] = sum_k h[b, t, k] * emb[v, k]  (bf16 products, fp32 sums)
 * of the shared LM head ([163], paragraph before the three-step pipeline),
 * which are reduced to per-128-token softmax partials on the fly and never
 * stored.  The residual draw finds its 128-token block from those partials
 * (the block's mass less min(p, q~) of its candidates) and recomputes that
 * block's 128 logits of row n (fp32 dot products, another summation order
 * than the matrix-core pass: a draw that falls within about 1e-6 of a
 * boundary may come out on its other side).
 *   h    [B, T+1, d] bf16; emb [vocab, d] bf16 (emb_dt = DF2_BF16), both
 *        16-byte aligned
 *   path_tok, path_rank [B, T]; cand_idx [B, T, K]; q [B, T, K]; seed_dev,
 *   b0, accept_len, out_tok, temperature: as in dflash2_verify_reject.
 * Limits: d % 64 == 0, d <= 65536, 1 <= T <= 63, 1 <= K <= 16, B <= 16384.
 * ws: block partials [B * (T+1), ceil(vocab / 128)] of 16 bytes plus small
 * per-row and per-request records, dflash2_verify_reject_head_workspace_bytes.
 * ------------------------------------------------------------------------ */
size_t dflash2_verify_reject_head_workspace_bytes(int B, int T, int64_t vocab, int d, int K);
int dflash2_verify_reject_head(const void* h, const void* emb, int emb_dt, int64_t vocab, int d,
                               const int32_t* path_tok, const int32_t* path_rank, const int32_t* cand_idx,
                               const float* q, int B, int T, int K, float temperature, const uint64_t* seed_dev,
                               int b0, int32_t* accept_len, int32_t* out_tok, void* ws, size_t ws_bytes,
                               hipStream_t stream);

/* ------------------------------------------------------------------------
 * One whole cycle of a small batch in one launch: dflash2_topk, then
 * dflash2_pair_scores, dflash2_path_viterbi (VITERBI or GREEDY) and
 * dflash2_verify_greedy on the same arguments, with the same results bit for
 * bit ([KDP] "A lightweight path selector"; [WC] 坑 6: at batch 1 decoding
 * speed is set by launch overhead).  The stages run as work-groups of one
 * launch that wait for each other through counters in the workspace instead
 * of kernel boundaries.
 *   logits [B, T, vocab] bf16 (drafter), target [B, T+1, vocab] bf16,
 *   emb [vocab, d], h [B, T, d], w_a, w_b, w_h [r, d] bf16, last_tok [B],
 *   gate: as dflash2_pair_scores; path_mode: DF2_PATH_VITERBI or
 *   DF2_PATH_GREEDY.
 *   Outputs: cand_idx, cand_val [B, T, K]; scores [B, T, K, K]; path_rank,
 *   path_tok [B, T]; q [B, T, K]; path_score [B] (may be NULL); accept_len
 *   [B]; out_tok [B, T+1]; status [1] int32 (device): 0, 1 if a stage
 *   waited too long for another, 2 if the control words were not zero at
 *   the start (the outputs are then not valid).
 * Limits: B T <= 1024, 1 <= T <= 63, 1 <= K <= 16, d % 64 == 0, r % 16 == 0
 * in [16, 256]; vocab * d * 2 < 2^32.
 * ws: dflash2_cycle_fused_workspace_bytes.  Its control words must be zero
 * before the first call: call dflash2_cycle_fused_init once after allocating
 * it (every call leaves them zero again).  Calls that share a workspace must
 * be ordered on one stream.
 * ------------------------------------------------------------------------ */
size_t dflash2_cycle_fused_workspace_bytes(int B, int T, int K, int64_t vocab, int d, int r);
int dflash2_cycle_fused_init(int B, int T, int K, int64_t vocab, int d, int r, void* ws, size_t ws_bytes,
                             hipStream_t stream);
int dflash2_cycle_fused(const void* logits, int logits_dt, const void* target, int target_dt, int64_t vocab,
                        const void* emb, int emb_dt, const void* h, const void* w_a, const void* w_b,
                        const void* w_h, const int32_t* last_tok, int B, int T, int K, int d, int r, int gate,
                        int path_mode, int32_t* cand_idx, float* cand_val, float* scores, int32_t* path_rank,
                        int32_t* path_tok, float* q, float* path_score, int32_t* accept_len, int32_t* out_tok,
                        int32_t* status, void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Philox4x64-10 words as the sampling steps above draw them (Salmon et al.,
 * "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11): for each i,
 * out[4i..4i+3] = Philox4x64-10(key = (seed, 0), counter = (t[i], b[i], 0, 0)).
 *   seed_dev [1] uint64; b, t [n] int32; out [4n] uint64 (all device).
 * ------------------------------------------------------------------------ */
int dflash2_philox4x64(const uint64_t* seed_dev, const int32_t* b, const int32_t* t, int n,
                       uint64_t* out, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Kernel timing hook (host).  Arms this thread so that every later launch of
 * the kernel with tag `kernel` records a start and a stop HIP event in its
 * own dispatch (hipExtLaunchKernel: the interval of the kernel's dispatch,
 * without stream-side overhead), for at most max_launches launches.  Tags:
 *   "topk_chunk", "topk_merge", "project_gemm", "proj_reduce", "h_gemm",
 *   "table_gemm", "pair_epilogue", "path", "argmax_part", "greedy_final",
 *   "sumexp_part", "residual_fused", "residual_chunk", "residual_find", "conv_gemm",
 *   "conv_epilogue", "philox",
 *   "lmhead_topk", "lmhead_merge", "head_argmax", "greedy_head_final",
 *   "head_stats", "head_row_reduce", "head_decide", "head_block_logits",
 *   "head_draw", "cycle_fused", "fused_clear".
 * dflash2_profile_stop waits for the recorded events, writes up to `max`
 * per-launch durations in milliseconds to ms (host) and their count to *n,
 * and disarms.  Not for use during graph capture.  Events are created on
 * the first use and kept; no device memory is allocated.
 * ------------------------------------------------------------------------ */
int dflash2_profile_start(const char* kernel, int max_launches);
int dflash2_profile_stop(float* ms, int max, int* n);

#ifdef __cplusplus
}
#endif

#endif /* DFLASH2_H */

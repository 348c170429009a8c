// api.hip -- the C ABI (include/dflash2.h): argument validation on the host,
// workspace carving, launches on the caller's stream, status codes.
// No entry point allocates, synchronises or reads device memory.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <atomic>
#include <mutex>

#include "dflash2.h"
#include "df2_internal.h"
#include "cycle_fused.h"

using namespace df2;

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return status;
}

int hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) {
    g_err[0] = 0;
    return DF2_OK;
  }
  return fail(DF2_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_dt(int dt, const char* name) {
  if (dt != DF2_FP32 && dt != DF2_BF16 && dt != DF2_FP16)
    return fail(DF2_ERR_DTYPE, "%s: dtype %d is not a dense FP32/BF16/FP16 code", name, dt);
  return DF2_OK;
}

int elem_size(int dt) { return dt == DF2_FP32 ? 4 : 2; }

#define REQUIRE(cond, status, ...) \
  do {                             \
    if (!(cond)) return fail(status, __VA_ARGS__); \
  } while (0)

constexpr int kMaxT = 63;
constexpr int64_t kMaxVocab = (int64_t)1 << 31;
constexpr int kMaxB = 1 << 20;

}  // namespace

// Scratch of dflash2_verify_greedy_noalloc: a fixed device array, one copy
// per GPU, held until the process ends.  Host code never passes this name
// to a kernel (on the host it is only a stand-in for the symbol); it uses
// the device address that scratch_address() resolves for each device.
constexpr size_t kScratchBytes = (size_t)1 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
int scratch_address(void** out, const char* fn) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, fn);
  if (dev < 0 || dev >= kMaxDevices)
    return fail(DF2_ERR_UNSUPPORTED, "%s: device %d beyond the %d the library tracks", fn, dev, kMaxDevices);
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_status(e, fn);
      if (!p) return fail(DF2_ERR_HIP, "%s: no device address for the scratch array", fn);
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return DF2_OK;
}

}  // namespace

extern "C" {

int dflash2_abi_version(void) { return DFLASH2_ABI_VERSION; }

const char* dflash2_status_string(int status) {
  switch (status) {
    case DF2_OK: return "ok";
    case DF2_ERR_NULL: return "null pointer";
    case DF2_ERR_DTYPE: return "unsupported dtype";
    case DF2_ERR_SHAPE: return "size out of range";
    case DF2_ERR_WORKSPACE: return "workspace too small";
    case DF2_ERR_UNSUPPORTED: return "unsupported mode or temperature";
    case DF2_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* dflash2_last_error(void) { return g_err; }

int dflash2_init(void) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "dflash2_init");
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return hip_status(e, "dflash2_init");
  void* scratch_dev = nullptr;
  if (int st = scratch_address(&scratch_dev, "dflash2_init")) return st;
  g_err[0] = 0;
  return DF2_OK;
}

// ------------------------------------------------------------------ top-K
size_t dflash2_topk_workspace_bytes(int64_t rows, int64_t vocab, int k) {
  if (rows <= 0 || vocab <= 0) return 0;
  return topk_plan(rows, vocab, k).ws_bytes;
}

int dflash2_topk(const void* logits, int dt, int64_t rows, int64_t vocab, int k, int32_t* out_idx,
                 float* out_val, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_dt(dt, "dflash2_topk");
  if (st) return st;
  REQUIRE(rows >= 0, DF2_ERR_SHAPE, "dflash2_topk: rows %lld < 0", (long long)rows);
  REQUIRE(vocab >= 1 && vocab < kMaxVocab, DF2_ERR_SHAPE, "dflash2_topk: vocab %lld", (long long)vocab);
  REQUIRE(k >= 1 && k <= 16 && k <= vocab, DF2_ERR_SHAPE, "dflash2_topk: k %d not in [1, min(16, vocab)]", k);
  if (rows == 0) return DF2_OK;
  REQUIRE(logits && out_idx && out_val, DF2_ERR_NULL, "dflash2_topk: null logits/out_idx/out_val");
  REQUIRE(((uintptr_t)logits % elem_size(dt)) == 0, DF2_ERR_SHAPE, "dflash2_topk: misaligned logits");
  TopkPlan plan = topk_plan(rows, vocab, k);
  REQUIRE(plan.ws_bytes == 0 || (ws && ws_bytes >= plan.ws_bytes), DF2_ERR_WORKSPACE,
          "dflash2_topk: workspace %zu < %zu bytes", ws_bytes, plan.ws_bytes);
  return hip_status(launch_topk(logits, dt, rows, vocab, k, out_idx, out_val, ws, plan, stream),
                    "dflash2_topk");
}

// ------------------------------------------------------------------ LM head + top-K
size_t dflash2_lm_head_topk_workspace_bytes(int rows, int64_t vocab, int d, int k) {
  if (rows <= 0 || vocab <= 0 || d <= 0) return 0;
  (void)k;
  return lmhead_plan(rows, vocab, d, 16).ws_bytes;
}

int dflash2_lm_head_topk(const void* h, const void* emb, int emb_dt, int64_t vocab, int rows, int d, int k,
                         int32_t* out_idx, float* out_val, void* ws, size_t ws_bytes, hipStream_t stream) {
  REQUIRE(emb_dt == DF2_BF16, DF2_ERR_DTYPE, "dflash2_lm_head_topk: the LM head must be BF16");
  REQUIRE(rows >= 0 && rows <= kMaxB, DF2_ERR_SHAPE, "dflash2_lm_head_topk: rows %d", rows);
  REQUIRE(vocab >= 1 && vocab < kMaxVocab, DF2_ERR_SHAPE, "dflash2_lm_head_topk: vocab %lld", (long long)vocab);
  REQUIRE(d >= 64 && d % 64 == 0 && d <= 65536, DF2_ERR_SHAPE,
          "dflash2_lm_head_topk: d %d is not a multiple of 64 in [64, 65536]", d);
  REQUIRE(k >= 1 && k <= 16 && k <= vocab, DF2_ERR_SHAPE, "dflash2_lm_head_topk: k %d not in [1, min(16, vocab)]", k);
  if (rows == 0) return DF2_OK;
  REQUIRE(h && emb && out_idx && out_val, DF2_ERR_NULL, "dflash2_lm_head_topk: null pointer argument");
  REQUIRE(aligned16(h) && aligned16(emb), DF2_ERR_SHAPE, "dflash2_lm_head_topk: h/emb must be 16-byte aligned");
  LmHeadPlan plan = lmhead_plan(rows, vocab, d, 16);
  REQUIRE(ws && ws_bytes >= plan.ws_bytes, DF2_ERR_WORKSPACE, "dflash2_lm_head_topk: workspace %zu < %zu bytes",
          ws_bytes, plan.ws_bytes);
  return hip_status(launch_lmhead_topk(h, emb, vocab, rows, d, k, out_idx, out_val, ws, plan, stream),
                    "dflash2_lm_head_topk");
}

// ------------------------------------------------------------------ greedy verify from the head
size_t dflash2_verify_greedy_head_workspace_bytes(int B, int T, int64_t vocab, int d) {
  if (B <= 0 || T <= 0 || vocab <= 0 || d <= 0) return 0;
  return lmhead_plan(B * (T + 1), vocab, d, 1).ws_bytes;
}

int dflash2_verify_greedy_head(const void* h, const void* emb, int emb_dt, int64_t vocab, int d,
                               const int32_t* path_tok, int B, int T, int32_t* accept_len, int32_t* out_tok,
                               void* ws, size_t ws_bytes, hipStream_t stream) {
  REQUIRE(emb_dt == DF2_BF16, DF2_ERR_DTYPE, "dflash2_verify_greedy_head: the LM head must be BF16");
  REQUIRE(vocab >= 1 && vocab < kMaxVocab, DF2_ERR_SHAPE, "dflash2_verify_greedy_head: vocab %lld",
          (long long)vocab);
  REQUIRE(d >= 64 && d % 64 == 0 && d <= 65536, DF2_ERR_SHAPE,
          "dflash2_verify_greedy_head: d %d is not a multiple of 64 in [64, 65536]", d);
  REQUIRE(B >= 0 && B <= kMaxB / 64, DF2_ERR_SHAPE, "dflash2_verify_greedy_head: B %d", B);
  REQUIRE(T >= 1 && T <= kMaxT, DF2_ERR_SHAPE, "dflash2_verify_greedy_head: T %d not in [1, %d]", T, kMaxT);
  if (B == 0) return DF2_OK;
  REQUIRE(h && emb && path_tok && accept_len && out_tok, DF2_ERR_NULL,
          "dflash2_verify_greedy_head: null pointer argument");
  REQUIRE(aligned16(h) && aligned16(emb), DF2_ERR_SHAPE, "dflash2_verify_greedy_head: h/emb must be 16-byte aligned");
  LmHeadPlan plan = lmhead_plan(B * (T + 1), vocab, d, 1);
  REQUIRE(ws && ws_bytes >= plan.ws_bytes, DF2_ERR_WORKSPACE,
          "dflash2_verify_greedy_head: workspace %zu < %zu bytes", ws_bytes, plan.ws_bytes);
  return hip_status(launch_verify_greedy_head(h, emb, vocab, d, path_tok, B, T, accept_len, out_tok, ws, plan,
                                              stream),
                    "dflash2_verify_greedy_head");
}

size_t dflash2_verify_reject_head_workspace_bytes(int B, int T, int64_t vocab, int d, int K) {
  if (B <= 0 || T <= 0 || vocab <= 0 || d <= 0 || K <= 0) return 0;
  return head_reject_plan(B, T, vocab, d, K).ws_bytes;
}

int dflash2_verify_reject_head(const void* h, const void* emb, int emb_dt, int64_t vocab, int d,
                               const int32_t* path_tok, const int32_t* path_rank, const int32_t* cand_idx,
                               const float* q, int B, int T, int K, float temperature, const uint64_t* seed_dev,
                               int b0, int32_t* accept_len, int32_t* out_tok, void* ws, size_t ws_bytes,
                               hipStream_t stream) {
  REQUIRE(emb_dt == DF2_BF16, DF2_ERR_DTYPE, "dflash2_verify_reject_head: the LM head must be BF16");
  REQUIRE(temperature > 0.f && isfinite(temperature), DF2_ERR_UNSUPPORTED,
          "dflash2_verify_reject_head: needs a finite temperature > 0 (got %g)", (double)temperature);
  REQUIRE(vocab >= 1 && vocab < kMaxVocab, DF2_ERR_SHAPE, "dflash2_verify_reject_head: vocab %lld",
          (long long)vocab);
  REQUIRE(d >= 64 && d % 64 == 0 && d <= 65536, DF2_ERR_SHAPE,
          "dflash2_verify_reject_head: d %d is not a multiple of 64 in [64, 65536]", d);
  REQUIRE(B >= 0 && B <= kMaxB / 64, DF2_ERR_SHAPE, "dflash2_verify_reject_head: B %d", B);
  REQUIRE(T >= 1 && T <= kMaxT, DF2_ERR_SHAPE, "dflash2_verify_reject_head: T %d not in [1, %d]", T, kMaxT);
  REQUIRE(K >= 1 && K <= 16, DF2_ERR_SHAPE, "dflash2_verify_reject_head: K %d not in [1, 16]", K);
  REQUIRE(b0 >= 0 && (int64_t)b0 + B <= ((int64_t)1 << 31) - 1, DF2_ERR_SHAPE,
          "dflash2_verify_reject_head: b0 %d (with B %d) outside [0, 2^31 - 1]", b0, B);
  if (B == 0) return DF2_OK;
  REQUIRE(h && emb && path_tok && path_rank && cand_idx && q && seed_dev && accept_len && out_tok, DF2_ERR_NULL,
          "dflash2_verify_reject_head: null pointer argument");
  REQUIRE(aligned16(h) && aligned16(emb), DF2_ERR_SHAPE, "dflash2_verify_reject_head: h/emb must be 16-byte aligned");
  HeadRejectPlan plan = head_reject_plan(B, T, vocab, d, K);
  REQUIRE(ws && ws_bytes >= plan.ws_bytes, DF2_ERR_WORKSPACE,
          "dflash2_verify_reject_head: workspace %zu < %zu bytes", ws_bytes, plan.ws_bytes);
  return hip_status(launch_verify_reject_head(h, emb, vocab, d, path_tok, path_rank, cand_idx, q, B, T, K,
                                              temperature, seed_dev, b0, accept_len, out_tok, ws, plan, stream),
                    "dflash2_verify_reject_head");
}

// ------------------------------------------------------------------ pair scores
namespace {
// projection tiling: 128-row tiles, one work-group per CU, 8 waves (two per
// SIMD) in two alternating groups over 4 LDS stages.  In the batch-32 /
// block-16 cycle (replayed graph, top-K + pair scores + path + verify):
// 142.1 us with both groups in step over 3 stages against 144.7 us with 4
// waves over 4 stages and 143.9-145.2 us with 64-row tiles; the alternating
// groups then took the projection alone (warm caches) from 49.3 to 47.6 us.
constexpr GemmTiling kProjTiling{128, 128, 4, 8, 3};
// The projection's K split: with few tiles (small batches) the reduction
// over d is split so that up to about one work-group per CU takes part
// (slices of >= 4 K-tiles, at most kMaxProjSplit).  The slices are summed
// in a fixed order by a reduce pass spread over many work-groups before the
// pair epilogue, which gates H after the sum.
constexpr int kMaxProjSplit = 8;
constexpr int kMaxProjSplitSmall = 16;
constexpr GemmTiling kProjTilingSmall{64, 128, 3, 4, 1};
constexpr int kSmallProjRows = 1024;
int split_for(const GemmTiling& t, int maxs, int B, int T, int K, int d, int r) {
  const int bm = t.bm, bn = t.bn;
  auto tl = [&](int m, int n) { return ((m + bm - 1) / bm) * ((n + bn - 1) / bn); };
  const int tiles = tl(B * T * K, r) + tl(B * (T - 1) * K, r) + tl(B, r) + tl(B * T, r);
  int ks = 256 / (tiles > 0 ? tiles : 1);
  if (ks > d / 64 / 4) ks = d / 64 / 4;
  if (ks > maxs) ks = maxs;
  return ks < 1 ? 1 : ks;
}
// 64 x 128 tiles (4 waves, up to 16 slices) below 1,024 candidate rows,
// 128 x 128 from there on.  Per cycle: batch 1 / block 8 47.9 -> 45.8 us,
// batch 8 / block 8 sampled 96.5 -> 93.8.  With both waves of a SIMD in
// step the 64 x 128 tiles also won where they needed no K split while the
// 128 x 128 ones did (batch 32 / block 8, 3,584 rows: 94.4 -> 91.5); on the
// two alternating wave groups the 128 x 128 tiles with two slices win there
// (88.3-88.4 against 89.9-90.2 us).
bool proj_small(int B, int T, int K, int d, int r) {
  (void)d;
  (void)r;
  return B * T * K < kSmallProjRows;
}
// 256 x 128 tiles (three LDS stages, same loop) where the 128 x 128 ones
// need more than one round of work-groups: a quarter fewer operand bytes
// per work-group and one round.  64 requests, block 16 (484 tiles of 128 x
// 128 against 244): 822 -> 803 us per stress cycle; where they would need a
// K split instead (batch 32 / block 16: 124 tiles, two slices and a 12.5 us
// slice sum) they lost, 0.442 -> 0.450 ms.  The per-token table build
// (4,748 tiles of 128 x 128 at V = 151,936) takes them too: 1.05 -> 0.877 ms.
constexpr GemmTiling kProjTilingBig{256, 128, 3, 8, 3};
int proj_tiles(const GemmTiling& t, int B, int T, int K, int r) {
  auto tl = [&](int m, int n) { return ((m + t.bm - 1) / t.bm) * ((n + t.bn - 1) / t.bn); };
  return tl(B * T * K, r) + tl(B * (T - 1) * K, r) + tl(B, r) + tl(B * T, r);
}
const GemmTiling& proj_tiling(int B, int T, int K, int d, int r) {
  if (proj_small(B, T, K, d, r)) return kProjTilingSmall;
  return proj_tiles(kProjTiling, B, T, K, r) > 256 ? kProjTilingBig : kProjTiling;
}
int proj_split(int B, int T, int K, int d, int r) {
  const GemmTiling& t = proj_tiling(B, T, K, d, r);
  return split_for(t, &t == &kProjTilingSmall ? kMaxProjSplitSmall : kMaxProjSplit, B, T, K, d, r);
}
struct PairWs {
  int split;
  size_t ab, alast, h, total;       // per-slice sizes are [rows, cols] fp32
  size_t ab_k, alast_k, h_k;        // floats between slices
};
PairWs pair_ws(int B, int T, int K, int d, int r) {
  PairWs w;
  w.split = proj_split(B, T, K, d, r);
  w.ab_k = (size_t)B * T * K * 2 * r;
  w.alast_k = (size_t)B * r;
  w.h_k = (size_t)B * T * r;
  size_t off = 0;
  w.ab = off;
  off += align256(w.split * w.ab_k * sizeof(float));
  w.alast = off;
  off += align256(w.split * w.alast_k * sizeof(float));
  w.h = off;
  off += align256(w.split * w.h_k * sizeof(float));
  w.total = off;
  return w;
}
// The projection problems of the pair scores, in the order [B(cand),
// A(cand), A(last), H]: candidates' B = E[cand] W_B^T into columns r .. 2r-1
// of ab, their A (positions 0 .. T-2 only) into columns 0 .. r-1, A of the
// last verified tokens, and H = h W_H^T (the gate is applied by the epilogue).
void proj_segments(const int32_t* cand_idx, const int32_t* last_tok, const void* emb, int64_t vocab, const void* h,
                   const void* w_a, const void* w_b, const void* w_h, int B, int T, int K, int d, int r,
                   const PairWs& pw, float* ab, float* alast, float* hg, GemmSeg* s) {
  for (int i = 0; i < 4; ++i) s[i] = GemmSeg{};
  // candidates, B half: B = E[cand] W_B^T into columns r .. 2r - 1 of ab
  s[0].x = (const uint16_t*)emb;
  s[0].gather = cand_idx;
  s[0].x_rows = vocab;
  s[0].ldx = d;
  s[0].M = B * T * K;
  s[0].w0 = s[0].w1 = (const uint16_t*)w_b;
  s[0].n0 = r;
  s[0].N = r;
  s[0].out = ab + r;
  s[0].ldo = 2 * r;
  s[0].out_kstride = (int64_t)pw.ab_k;
  s[0].gate = DF2_GATE_IDENTITY;
  // candidates, A half: only positions 0 .. T-2 precede another position
  // (the last block position's A is never read), so the leading (T - 1) K
  // rows of every request's T K candidates (none when T = 1)
  s[1] = s[0];
  s[1].M = B * (T - 1) * K;
  s[1].grp_rows = (T - 1) * K;
  s[1].grp_stride = T * K;
  s[1].w0 = s[1].w1 = (const uint16_t*)w_a;
  s[1].out = ab;
  // last verified tokens: A only
  s[2] = s[0];
  s[2].gather = last_tok;
  s[2].M = B;
  s[2].w0 = s[2].w1 = (const uint16_t*)w_a;
  s[2].out = alast;
  s[2].ldo = r;
  s[2].out_kstride = (int64_t)pw.alast_k;
  // gate: H = gate(h W_H^T), the gate applied by the epilogue
  s[3].x = (const uint16_t*)h;
  s[3].gather = nullptr;
  s[3].x_rows = (int64_t)B * T;
  s[3].ldx = d;
  s[3].M = B * T;
  s[3].w0 = (const uint16_t*)w_h;
  s[3].w1 = (const uint16_t*)w_h;
  s[3].n0 = r;
  s[3].N = r;
  s[3].out = hg;
  s[3].ldo = r;
  s[3].out_kstride = (int64_t)pw.h_k;
  s[3].gate = DF2_GATE_IDENTITY;
}
}  // namespace

size_t dflash2_pair_scores_workspace_bytes(int B, int T, int K, int d, int r) {
  if (B <= 0 || T <= 0 || K <= 0 || r <= 0 || d < 64) return 0;
  return pair_ws(B, T, K, d, r).total;
}

int dflash2_pair_scores(const int32_t* cand_idx, const float* cand_val, const int32_t* last_tok,
                        const void* emb, int emb_dt, int64_t vocab, const void* h, const void* w_a,
                        const void* w_b, const void* w_h, int B, int T, int K, int d, int r,
                        int gate, float* scores, void* ws, size_t ws_bytes, hipStream_t stream) {
  REQUIRE(emb_dt == DF2_BF16, DF2_ERR_DTYPE, "dflash2_pair_scores: embedding table must be BF16");
  REQUIRE(B >= 0 && B <= kMaxB, DF2_ERR_SHAPE, "dflash2_pair_scores: B %d", B);
  REQUIRE(T >= 1 && T <= kMaxT, DF2_ERR_SHAPE, "dflash2_pair_scores: T %d not in [1, %d]", T, kMaxT);
  REQUIRE(K >= 1 && K <= 16, DF2_ERR_SHAPE, "dflash2_pair_scores: K %d not in [1, 16]", K);
  REQUIRE(d >= 64 && d % 64 == 0, DF2_ERR_SHAPE, "dflash2_pair_scores: d %d is not a positive multiple of 64", d);
  REQUIRE(r >= 16 && r <= 256 && r % 16 == 0, DF2_ERR_SHAPE, "dflash2_pair_scores: r %d not a multiple of 16 in [16, 256]", r);
  REQUIRE(vocab >= 1 && vocab < kMaxVocab, DF2_ERR_SHAPE, "dflash2_pair_scores: vocab %lld", (long long)vocab);
  REQUIRE((uint64_t)vocab * (uint64_t)d * 2u < (1ull << 32), DF2_ERR_UNSUPPORTED,
          "dflash2_pair_scores: embedding table of %lld x %d bf16 is 4 GiB or more", (long long)vocab, d);
  REQUIRE(gate == DF2_GATE_IDENTITY || gate == DF2_GATE_SIGMOID, DF2_ERR_UNSUPPORTED, "dflash2_pair_scores: gate %d", gate);
  if (B == 0) return DF2_OK;
  REQUIRE(cand_idx && cand_val && last_tok && emb && h && w_a && w_b && w_h && scores, DF2_ERR_NULL,
          "dflash2_pair_scores: null pointer argument");
  REQUIRE(aligned16(emb) && aligned16(h) && aligned16(w_a) && aligned16(w_b) && aligned16(w_h),
          DF2_ERR_SHAPE, "dflash2_pair_scores: emb/h/w_* must be 16-byte aligned");
  PairWs pw = pair_ws(B, T, K, d, r);
  REQUIRE(ws && ws_bytes >= pw.total, DF2_ERR_WORKSPACE, "dflash2_pair_scores: workspace %zu < %zu bytes",
          ws_bytes, pw.total);
  float* ab = (float*)((char*)ws + pw.ab);
  float* alast = (float*)((char*)ws + pw.alast);
  float* hg = (float*)((char*)ws + pw.h);
  GemmSeg s[4];
  proj_segments(cand_idx, last_tok, emb, vocab, h, w_a, w_b, w_h, B, T, K, d, r, pw, ab, alast, hg, s);
  hipError_t e = launch_gemm(s, 4, d, pw.split, proj_tiling(B, T, K, d, r), "project_gemm", stream);
  if (e != hipSuccess) return hip_status(e, "dflash2_pair_scores (projection)");
  return hip_status(launch_pair_epilogue(ab, alast, hg, pw.split, (int64_t)pw.ab_k, (int64_t)pw.alast_k,
                                         (int64_t)pw.h_k, gate, cand_val, B, T, K, r, scores, stream),
                    "dflash2_pair_scores (epilogue)");
}

// ------------------------------------------------------------------ fused small-batch cycle
namespace {
struct FusedWs {
  TopkPlan tp;
  int vsplits;
  int64_t vchunk;
  PairWs pw;
  size_t off_tpart, off_pair, off_vpart, off_ctr, total;
};
FusedWs fused_ws(int B, int T, int K, int64_t vocab, int d, int r) {
  FusedWs w;
  w.tp = fused_topk_plan((int64_t)B * T, vocab, K);
  w.vsplits = fused_verify_splits(B, T, vocab, w.vchunk);
  w.pw = pair_ws(B, T, K, d, r);
  size_t off = 0;
  w.off_tpart = off;
  off += align256(w.tp.ws_bytes);
  w.off_pair = off;
  off += align256(w.pw.total);
  w.off_vpart = off;
  off += align256((size_t)B * (T + 1) * w.vsplits * sizeof(uint64_t));
  w.off_ctr = off;
  off += align256(fused_ctr_bytes(B * T));
  w.total = off;
  return w;
}
constexpr int kMaxFusedRows = 1024;   // B * T
}  // namespace

size_t dflash2_cycle_fused_workspace_bytes(int B, int T, int K, int64_t vocab, int d, int r) {
  if (B <= 0 || T <= 0 || K <= 0 || vocab <= 0 || d < 64 || r <= 0) return 0;
  return fused_ws(B, T, K, vocab, d, r).total;
}

int dflash2_cycle_fused_init(int B, int T, int K, int64_t vocab, int d, int r, void* ws, size_t ws_bytes,
                             hipStream_t stream) {
  REQUIRE(B >= 0 && T >= 1 && T <= kMaxT && (int64_t)B * T <= kMaxFusedRows && K >= 1 && K <= 16 && d >= 64 &&
              r >= 16 && vocab >= 1 && vocab < kMaxVocab,
          DF2_ERR_SHAPE, "dflash2_cycle_fused_init: shape B %d T %d K %d d %d r %d", B, T, K, d, r);
  if (B == 0) return DF2_OK;
  FusedWs w = fused_ws(B, T, K, vocab, d, r);
  REQUIRE(ws && ws_bytes >= w.total, DF2_ERR_WORKSPACE, "dflash2_cycle_fused_init: workspace %zu < %zu bytes",
          ws_bytes, w.total);
  return hip_status(launch_fused_ctr_clear((char*)ws + w.off_ctr, B * T, stream), "dflash2_cycle_fused_init");
}

int dflash2_cycle_fused(const void* logits, int logits_dt, const void* target, int target_dt, int64_t vocab,
                        const void* emb, int emb_dt, const void* h, const void* w_a, const void* w_b,
                        const void* w_h, const int32_t* last_tok, int B, int T, int K, int d, int r, int gate,
                        int path_mode, int32_t* cand_idx, float* cand_val, float* scores, int32_t* path_rank,
                        int32_t* path_tok, float* q, float* path_score, int32_t* accept_len, int32_t* out_tok,
                        int32_t* status, void* ws, size_t ws_bytes, hipStream_t stream) {
  REQUIRE(logits_dt == DF2_BF16 && target_dt == DF2_BF16 && emb_dt == DF2_BF16, DF2_ERR_DTYPE,
          "dflash2_cycle_fused: logits, target logits and embedding table must be BF16");
  REQUIRE(path_mode == DF2_PATH_VITERBI || path_mode == DF2_PATH_GREEDY, DF2_ERR_UNSUPPORTED,
          "dflash2_cycle_fused: path mode %d (VITERBI or GREEDY)", path_mode);
  REQUIRE(gate == DF2_GATE_IDENTITY || gate == DF2_GATE_SIGMOID, DF2_ERR_UNSUPPORTED, "dflash2_cycle_fused: gate %d",
          gate);
  REQUIRE(B >= 0 && T >= 1 && T <= kMaxT && (int64_t)B * T <= kMaxFusedRows, DF2_ERR_SHAPE,
          "dflash2_cycle_fused: B %d T %d (1 <= T <= %d, B T <= %d)", B, T, kMaxT, kMaxFusedRows);
  REQUIRE(K >= 1 && K <= 16, DF2_ERR_SHAPE, "dflash2_cycle_fused: K %d not in [1, 16]", K);
  REQUIRE(d >= 64 && d % 64 == 0, DF2_ERR_SHAPE, "dflash2_cycle_fused: d %d is not a positive multiple of 64", d);
  REQUIRE(r >= 16 && r <= 256 && r % 16 == 0, DF2_ERR_SHAPE,
          "dflash2_cycle_fused: r %d not a multiple of 16 in [16, 256]", r);
  REQUIRE(vocab >= 1 && vocab < kMaxVocab, DF2_ERR_SHAPE, "dflash2_cycle_fused: vocab %lld", (long long)vocab);
  REQUIRE((uint64_t)vocab * (uint64_t)d * 2u < (1ull << 32), DF2_ERR_UNSUPPORTED,
          "dflash2_cycle_fused: embedding table of %lld x %d bf16 is 4 GiB or more", (long long)vocab, d);
  if (B == 0) return DF2_OK;
  REQUIRE(logits && target && emb && h && w_a && w_b && w_h && last_tok && cand_idx && cand_val && scores &&
              path_rank && path_tok && q && accept_len && out_tok && status,
          DF2_ERR_NULL, "dflash2_cycle_fused: null pointer argument");
  REQUIRE(aligned16(emb) && aligned16(h) && aligned16(w_a) && aligned16(w_b) && aligned16(w_h) && aligned16(scores),
          DF2_ERR_SHAPE, "dflash2_cycle_fused: emb/h/w_*/scores must be 16-byte aligned");
  FusedWs w = fused_ws(B, T, K, vocab, d, r);
  REQUIRE(ws && ws_bytes >= w.total, DF2_ERR_WORKSPACE, "dflash2_cycle_fused: workspace %zu < %zu bytes", ws_bytes,
          w.total);
  char* base = (char*)ws;
  float* ab = (float*)(base + w.off_pair + w.pw.ab);
  float* alast = (float*)(base + w.off_pair + w.pw.alast);
  float* hg = (float*)(base + w.off_pair + w.pw.h);
  GemmSeg s[4], f[4];
  proj_segments(cand_idx, last_tok, emb, vocab, h, w_a, w_b, w_h, B, T, K, d, r, w.pw, ab, alast, hg, s);
  f[0] = s[2];   // A(last) and H first: they need no candidates
  f[1] = s[3];
  f[2] = s[0];
  f[3] = s[1];
  FusedArgs a{};
  a.logits = logits;
  a.target = target;
  a.vocab = vocab;
  a.B = B;
  a.T = T;
  a.K = K;
  a.r = r;
  a.gate = gate;
  a.mode = path_mode;
  a.tsplits = w.tp.splits;
  a.tchunk = w.tp.chunk;
  a.tpart = (uint64_t*)(base + w.off_tpart);
  a.cand_idx = cand_idx;
  a.cand_val = cand_val;
  a.P.ksplit = w.pw.split;
  a.ab = ab;
  a.alast = alast;
  a.hg = hg;
  a.ab_k = (int64_t)w.pw.ab_k;
  a.alast_k = (int64_t)w.pw.alast_k;
  a.h_k = (int64_t)w.pw.h_k;
  a.n0 = (int64_t)B * T * K * 2 * r / 4;
  a.n1 = (int64_t)B * r / 4;
  a.n2 = (int64_t)B * T * r / 4;
  a.scores = scores;
  a.path_rank = path_rank;
  a.path_tok = path_tok;
  a.q = q;
  a.path_score = path_score;
  a.vsplits = w.vsplits;
  a.vchunk = w.vchunk;
  a.vpart = (uint64_t*)(base + w.off_vpart);
  a.accept_len = accept_len;
  a.out_tok = out_tok;
  a.ctr = (uint32_t*)(base + w.off_ctr);
  a.status = status;
  return hip_status(launch_cycle_fused(a, f, d, stream), "dflash2_cycle_fused");
}

// ------------------------------------------------------------------ per-token tables
// A(tok) and B(tok) depend on the token alone, so [A | B] can be computed
// once for the whole vocabulary: one GEMM E [W_A; W_B]^T with thousands of
// tiles and no split of the reduction over d.
int dflash2_selector_tables(const void* emb, int emb_dt, int64_t vocab, int d, const void* w_a,
                            const void* w_b, int r, float* tab, hipStream_t stream) {
  REQUIRE(emb_dt == DF2_BF16, DF2_ERR_DTYPE, "dflash2_selector_tables: embedding table must be BF16");
  REQUIRE(d >= 64 && d % 64 == 0, DF2_ERR_SHAPE, "dflash2_selector_tables: d %d is not a positive multiple of 64", d);
  REQUIRE(r >= 16 && r <= 256 && r % 16 == 0, DF2_ERR_SHAPE, "dflash2_selector_tables: r %d not a multiple of 16 in [16, 256]", r);
  REQUIRE(vocab >= 0 && vocab < kMaxVocab, DF2_ERR_SHAPE, "dflash2_selector_tables: vocab %lld", (long long)vocab);
  REQUIRE((uint64_t)vocab * (uint64_t)d * 2u < (1ull << 32), DF2_ERR_UNSUPPORTED,
          "dflash2_selector_tables: embedding table of %lld x %d bf16 is 4 GiB or more", (long long)vocab, d);
  if (vocab == 0) return DF2_OK;
  REQUIRE(emb && w_a && w_b && tab, DF2_ERR_NULL, "dflash2_selector_tables: null pointer argument");
  REQUIRE(aligned16(emb) && aligned16(w_a) && aligned16(w_b) && aligned16(tab), DF2_ERR_SHAPE,
          "dflash2_selector_tables: emb/w_a/w_b/tab must be 16-byte aligned");
  GemmSeg s[2] = {};
  s[0].x = (const uint16_t*)emb;
  s[0].gather = nullptr;
  s[0].x_rows = vocab;
  s[0].ldx = d;
  s[0].M = (int)vocab;
  s[0].w0 = (const uint16_t*)w_a;
  s[0].w1 = (const uint16_t*)w_b;
  s[0].n0 = r;
  s[0].N = 2 * r;
  s[0].out = tab;
  s[0].ldo = 2 * r;
  s[0].out_kstride = 0;
  s[0].gate = DF2_GATE_IDENTITY;
  int nseg = 1;
  if (r % 128 != 0) {   // W tiles may not straddle W_A / W_B
    s[1] = s[0];
    s[0].w1 = s[0].w0;
    s[0].N = r;
    s[1].w0 = s[1].w1 = (const uint16_t*)w_b;
    s[1].N = r;
    s[1].out = tab + r;
    nseg = 2;
  }
  return hip_status(launch_gemm(s, nseg, d, 1, kProjTilingBig, "table_gemm", stream), "dflash2_selector_tables");
}

namespace {
// Per cycle only H = W_H h is projected: B*T rows, a skinny product whose
// reduction over d is split so that about one work-group per CU takes part
// (64 x 128 tiles; slices of >= 4 K-tiles, at most kMaxHSplit); the
// table-mode pair epilogue sums the slices in slice order itself.
constexpr GemmTiling kHTiling{64, 128, 3, 4, 1};
constexpr int kMaxHSplit = 16;
int h_split(int B, int T, int d, int r) {
  const int tiles = ((B * T + kHTiling.bm - 1) / kHTiling.bm) * ((r + kHTiling.bn - 1) / kHTiling.bn);
  int ks = 256 / (tiles > 0 ? tiles : 1);
  if (ks > d / 64 / 4) ks = d / 64 / 4;
  if (ks > kMaxHSplit) ks = kMaxHSplit;
  return ks < 1 ? 1 : ks;
}
}  // namespace

size_t dflash2_pair_scores_tab_workspace_bytes(int B, int T, int d, int r) {
  if (B <= 0 || T <= 0 || r <= 0 || d < 64) return 0;
  return align256((size_t)h_split(B, T, d, r) * (size_t)B * T * r * sizeof(float));
}

namespace {
int check_tab_shapes(const char* fn, int B, int T, int K, int d, int r, int64_t vocab, int gate) {
  REQUIRE(B >= 0 && B <= kMaxB, DF2_ERR_SHAPE, "%s: B %d", fn, B);
  REQUIRE(T >= 1 && T <= kMaxT, DF2_ERR_SHAPE, "%s: T %d not in [1, %d]", fn, T, kMaxT);
  REQUIRE(K >= 1 && K <= 16, DF2_ERR_SHAPE, "%s: K %d not in [1, 16]", fn, K);
  REQUIRE(d >= 64 && d % 64 == 0, DF2_ERR_SHAPE, "%s: d %d is not a positive multiple of 64", fn, d);
  REQUIRE(r >= 16 && r <= 256 && r % 16 == 0, DF2_ERR_SHAPE, "%s: r %d not a multiple of 16 in [16, 256]", fn, r);
  REQUIRE(vocab >= 1 && vocab < kMaxVocab, DF2_ERR_SHAPE, "%s: vocab %lld", fn, (long long)vocab);
  REQUIRE(gate == DF2_GATE_IDENTITY || gate == DF2_GATE_SIGMOID, DF2_ERR_UNSUPPORTED, "%s: gate %d", fn, gate);
  return DF2_OK;
}

// H's split-K partial products (ungated) into ws.
hipError_t project_h(const void* h, const void* w_h, int B, int T, int d, int r, float* hg, hipStream_t stream) {
  GemmSeg s = {};
  s.x = (const uint16_t*)h;
  s.gather = nullptr;
  s.x_rows = (int64_t)B * T;
  s.ldx = d;
  s.M = B * T;
  s.w0 = (const uint16_t*)w_h;
  s.w1 = (const uint16_t*)w_h;
  s.n0 = r;
  s.N = r;
  s.out = hg;
  s.ldo = r;
  s.out_kstride = (int64_t)B * T * r;
  s.gate = DF2_GATE_IDENTITY;
  return launch_gemm(&s, 1, d, h_split(B, T, d, r), kHTiling, "h_gemm", stream);
}
}  // namespace

int dflash2_h_projection(const void* h, const void* w_h, int B, int T, int d, int r, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
  if (int st = check_tab_shapes("dflash2_h_projection", B, T, 1, d, r, 1, DF2_GATE_IDENTITY)) return st;
  if (B == 0) return DF2_OK;
  REQUIRE(h && w_h, DF2_ERR_NULL, "dflash2_h_projection: null pointer argument");
  REQUIRE(aligned16(h) && aligned16(w_h), DF2_ERR_SHAPE, "dflash2_h_projection: h/w_h must be 16-byte aligned");
  const size_t need = dflash2_pair_scores_tab_workspace_bytes(B, T, d, r);
  REQUIRE(ws && ws_bytes >= need, DF2_ERR_WORKSPACE, "dflash2_h_projection: workspace %zu < %zu bytes",
          ws_bytes, need);
  return hip_status(project_h(h, w_h, B, T, d, r, (float*)ws, stream), "dflash2_h_projection");
}

int dflash2_pair_scores_tab_from_h(const int32_t* cand_idx, const float* cand_val, const int32_t* last_tok,
                                   const float* tab, int64_t vocab, int B, int T, int K, int d, int r, int gate,
                                   float* scores, const void* ws, size_t ws_bytes, hipStream_t stream) {
  if (int st = check_tab_shapes("dflash2_pair_scores_tab_from_h", B, T, K, d, r, vocab, gate)) return st;
  if (B == 0) return DF2_OK;
  REQUIRE(cand_idx && cand_val && last_tok && tab && scores, DF2_ERR_NULL,
          "dflash2_pair_scores_tab_from_h: null pointer argument");
  REQUIRE(aligned16(tab), DF2_ERR_SHAPE, "dflash2_pair_scores_tab_from_h: tab must be 16-byte aligned");
  const size_t need = dflash2_pair_scores_tab_workspace_bytes(B, T, d, r);
  REQUIRE(ws && ws_bytes >= need, DF2_ERR_WORKSPACE, "dflash2_pair_scores_tab_from_h: workspace %zu < %zu bytes",
          ws_bytes, need);
  return hip_status(launch_pair_epilogue_tab(tab, vocab, cand_idx, last_tok, (const float*)ws, h_split(B, T, d, r),
                                             (int64_t)B * T * r, gate, cand_val, B, T, K, r, scores, stream),
                    "dflash2_pair_scores_tab_from_h");
}

int dflash2_pair_scores_tab(const int32_t* cand_idx, const float* cand_val, const int32_t* last_tok,
                            const float* tab, int64_t vocab, const void* h, const void* w_h, int B, int T,
                            int K, int d, int r, int gate, float* scores, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
  if (int st = check_tab_shapes("dflash2_pair_scores_tab", B, T, K, d, r, vocab, gate)) return st;
  if (B == 0) return DF2_OK;
  REQUIRE(cand_idx && cand_val && last_tok && tab && h && w_h && scores, DF2_ERR_NULL,
          "dflash2_pair_scores_tab: null pointer argument");
  REQUIRE(aligned16(tab) && aligned16(h) && aligned16(w_h), DF2_ERR_SHAPE,
          "dflash2_pair_scores_tab: tab/h/w_h must be 16-byte aligned");
  const size_t need = dflash2_pair_scores_tab_workspace_bytes(B, T, d, r);
  REQUIRE(ws && ws_bytes >= need, DF2_ERR_WORKSPACE, "dflash2_pair_scores_tab: workspace %zu < %zu bytes",
          ws_bytes, need);
  hipError_t e = project_h(h, w_h, B, T, d, r, (float*)ws, stream);
  if (e != hipSuccess) return hip_status(e, "dflash2_pair_scores_tab (projection)");
  return hip_status(launch_pair_epilogue_tab(tab, vocab, cand_idx, last_tok, (float*)ws, h_split(B, T, d, r),
                                             (int64_t)B * T * r, gate, cand_val, B, T, K, r, scores, stream),
                    "dflash2_pair_scores_tab (epilogue)");
}

// ------------------------------------------------------------------ path
int dflash2_path_viterbi(const float* scores, const int32_t* cand_idx, int B, int T, int K, int mode,
                         float temperature, const uint64_t* seed_dev, int b0, int32_t* path_rank,
                         int32_t* path_tok, float* q, float* path_score, hipStream_t stream) {
  REQUIRE(mode == DF2_PATH_VITERBI || mode == DF2_PATH_GREEDY || mode == DF2_PATH_SAMPLE,
          DF2_ERR_UNSUPPORTED, "dflash2_path_viterbi: mode %d", mode);
  REQUIRE(mode != DF2_PATH_SAMPLE || (temperature > 0.f && isfinite(temperature)), DF2_ERR_UNSUPPORTED,
          "dflash2_path_viterbi: sampling needs a finite temperature > 0 (got %g)", (double)temperature);
  REQUIRE(B >= 0 && B <= kMaxB, DF2_ERR_SHAPE, "dflash2_path_viterbi: B %d", B);
  REQUIRE(T >= 1 && T <= kMaxT, DF2_ERR_SHAPE, "dflash2_path_viterbi: T %d not in [1, %d]", T, kMaxT);
  REQUIRE(K >= 1 && K <= 16, DF2_ERR_SHAPE, "dflash2_path_viterbi: K %d not in [1, 16]", K);
  REQUIRE(b0 >= 0 && (int64_t)b0 + B <= ((int64_t)1 << 31) - 1, DF2_ERR_SHAPE,
          "dflash2_path_viterbi: b0 %d (with B %d) outside [0, 2^31 - 1]", b0, B);
  if (B == 0) return DF2_OK;
  REQUIRE(scores && cand_idx && path_rank && path_tok && q, DF2_ERR_NULL,
          "dflash2_path_viterbi: null pointer argument");
  REQUIRE(mode != DF2_PATH_SAMPLE || seed_dev, DF2_ERR_NULL, "dflash2_path_viterbi: sampling needs seed_dev");
  return hip_status(launch_path(scores, cand_idx, B, T, K, mode, temperature, seed_dev, b0, path_rank,
                                path_tok, q, path_score, stream),
                    "dflash2_path_viterbi");
}

// ------------------------------------------------------------------ dynconv2
size_t dflash2_dynconv2_workspace_bytes(int B, int L, int d, int group) {
  if (B <= 0 || L <= 0 || d <= 0 || group != 16 || d % 64) return 0;
  return conv_plan(B, L, d, group).ws_bytes;
}

int dflash2_dynconv2(const void* x, const void* x_prev, const void* w, const float* base, int B,
                     int L, int d, int group, void* y, int y_dt, void* ws, size_t ws_bytes,
                     hipStream_t stream) {
  REQUIRE(y_dt == DF2_BF16 || y_dt == DF2_FP32, DF2_ERR_DTYPE, "dflash2_dynconv2: y dtype %d", y_dt);
  REQUIRE(group == 16, DF2_ERR_SHAPE, "dflash2_dynconv2: group %d (only 16 is supported)", group);
  REQUIRE(d >= 64 && d % 64 == 0 && d <= 16384, DF2_ERR_SHAPE, "dflash2_dynconv2: d %d", d);
  REQUIRE(B >= 0 && L >= 1 && (int64_t)B * L < (1 << 30), DF2_ERR_SHAPE, "dflash2_dynconv2: B %d L %d", B, L);
  if (B == 0) return DF2_OK;
  REQUIRE(x && w && y, DF2_ERR_NULL, "dflash2_dynconv2: null x/w/y");
  REQUIRE(aligned16(x) && aligned16(w) && aligned16(y) && (!x_prev || aligned16(x_prev)), DF2_ERR_SHAPE,
          "dflash2_dynconv2: x/x_prev/w/y must be 16-byte aligned");
  ConvPlan plan = conv_plan(B, L, d, group);
  REQUIRE(ws && ws_bytes >= plan.ws_bytes, DF2_ERR_WORKSPACE, "dflash2_dynconv2: workspace %zu < %zu bytes",
          ws_bytes, plan.ws_bytes);
  return hip_status(launch_dynconv2(x, x_prev, w, base, B, L, d, group, y, y_dt == DF2_BF16 ? 1 : 0, ws,
                                    plan, stream),
                    "dflash2_dynconv2");
}

// ------------------------------------------------------------------ verify
size_t dflash2_verify_workspace_bytes(int B, int T, int64_t vocab) {
  if (B <= 0 || T <= 0 || vocab <= 0) return 0;
  return verify_plan(B, T, vocab).ws_bytes;
}

int dflash2_verify_greedy(const void* target_logits, int dt, int64_t vocab, const int32_t* path_tok,
                          int B, int T, int32_t* accept_len, int32_t* out_tok, void* ws,
                          size_t ws_bytes, hipStream_t stream) {
  int st = check_dt(dt, "dflash2_verify_greedy");
  if (st) return st;
  REQUIRE(vocab >= 1 && vocab < kMaxVocab, DF2_ERR_SHAPE, "dflash2_verify_greedy: vocab %lld", (long long)vocab);
  REQUIRE(B >= 0 && B <= kMaxB, DF2_ERR_SHAPE, "dflash2_verify_greedy: B %d", B);
  REQUIRE(T >= 1 && T <= kMaxT, DF2_ERR_SHAPE, "dflash2_verify_greedy: T %d not in [1, %d]", T, kMaxT);
  if (B == 0) return DF2_OK;
  REQUIRE(target_logits && path_tok && accept_len && out_tok, DF2_ERR_NULL,
          "dflash2_verify_greedy: null pointer argument");
  REQUIRE(((uintptr_t)target_logits % elem_size(dt)) == 0, DF2_ERR_SHAPE, "dflash2_verify_greedy: misaligned logits");
  VerifyPlan plan = verify_plan(B, T, vocab);
  REQUIRE(ws && ws_bytes >= plan.ws_bytes, DF2_ERR_WORKSPACE, "dflash2_verify_greedy: workspace %zu < %zu bytes",
          ws_bytes, plan.ws_bytes);
  return hip_status(launch_verify_greedy(target_logits, dt, vocab, path_tok, B, T, accept_len, out_tok,
                                         ws, plan, stream),
                    "dflash2_verify_greedy");
}

size_t dflash2_verify_greedy_noalloc_max_bytes(void) { return kScratchBytes; }

int dflash2_verify_greedy_noalloc(const void* target_logits, int dt, int64_t vocab, const int32_t* path_tok,
                                  int B, int T, int32_t* accept_len, int32_t* out_tok, hipStream_t stream) {
  int st = check_dt(dt, "dflash2_verify_greedy_noalloc");
  if (st) return st;
  REQUIRE(vocab >= 1 && vocab < kMaxVocab, DF2_ERR_SHAPE, "dflash2_verify_greedy_noalloc: vocab %lld",
          (long long)vocab);
  REQUIRE(B >= 0 && B <= kMaxB, DF2_ERR_SHAPE, "dflash2_verify_greedy_noalloc: B %d", B);
  REQUIRE(T >= 1 && T <= kMaxT, DF2_ERR_SHAPE, "dflash2_verify_greedy_noalloc: T %d not in [1, %d]", T, kMaxT);
  if (B == 0) return DF2_OK;
  REQUIRE(target_logits && path_tok && accept_len && out_tok, DF2_ERR_NULL,
          "dflash2_verify_greedy_noalloc: null pointer argument");
  REQUIRE(((uintptr_t)target_logits % elem_size(dt)) == 0, DF2_ERR_SHAPE,
          "dflash2_verify_greedy_noalloc: misaligned logits");
  VerifyPlan plan = verify_plan(B, T, vocab);
  REQUIRE(plan.ws_bytes <= kScratchBytes, DF2_ERR_WORKSPACE,
          "dflash2_verify_greedy_noalloc: this size needs %zu bytes of scratch, more than the fixed %zu "
          "(use dflash2_verify_greedy with a workspace)", plan.ws_bytes, kScratchBytes);
  void* ws = nullptr;
  if (int st2 = scratch_address(&ws, "dflash2_verify_greedy_noalloc")) return st2;
  // the kernels write every partial result before they read it: nothing
  // in the scratch has to start at zero
  return hip_status(launch_verify_greedy(target_logits, dt, vocab, path_tok, B, T, accept_len, out_tok,
                                         ws, plan, stream),
                    "dflash2_verify_greedy_noalloc");
}

int dflash2_verify_reject(const void* target_logits, int dt, int64_t vocab, const int32_t* path_tok,
                          const int32_t* path_rank, const int32_t* cand_idx, const float* q, int B,
                          int T, int K, float temperature, const uint64_t* seed_dev, int b0,
                          int32_t* accept_len, int32_t* out_tok, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
  int st = check_dt(dt, "dflash2_verify_reject");
  if (st) return st;
  REQUIRE(temperature > 0.f && isfinite(temperature), DF2_ERR_UNSUPPORTED,
          "dflash2_verify_reject: needs a finite temperature > 0 (got %g)", (double)temperature);
  REQUIRE(vocab >= 1 && vocab < kMaxVocab, DF2_ERR_SHAPE, "dflash2_verify_reject: vocab %lld", (long long)vocab);
  REQUIRE(B >= 0 && B <= kMaxB, DF2_ERR_SHAPE, "dflash2_verify_reject: B %d", B);
  REQUIRE(T >= 1 && T <= kMaxT, DF2_ERR_SHAPE, "dflash2_verify_reject: T %d not in [1, %d]", T, kMaxT);
  REQUIRE(K >= 1 && K <= 16, DF2_ERR_SHAPE, "dflash2_verify_reject: K %d not in [1, 16]", K);
  REQUIRE(b0 >= 0 && (int64_t)b0 + B <= ((int64_t)1 << 31) - 1, DF2_ERR_SHAPE,
          "dflash2_verify_reject: b0 %d (with B %d) outside [0, 2^31 - 1]", b0, B);
  if (B == 0) return DF2_OK;
  REQUIRE(target_logits && path_tok && path_rank && cand_idx && q && seed_dev && accept_len && out_tok,
          DF2_ERR_NULL, "dflash2_verify_reject: null pointer argument");
  REQUIRE(((uintptr_t)target_logits % elem_size(dt)) == 0, DF2_ERR_SHAPE, "dflash2_verify_reject: misaligned logits");
  VerifyPlan plan = verify_plan(B, T, vocab);
  REQUIRE(ws && ws_bytes >= plan.ws_bytes, DF2_ERR_WORKSPACE, "dflash2_verify_reject: workspace %zu < %zu bytes",
          ws_bytes, plan.ws_bytes);
  return hip_status(launch_verify_reject(target_logits, dt, vocab, path_tok, path_rank, cand_idx, q, B, T,
                                         K, temperature, seed_dev, b0, accept_len, out_tok, ws, plan, stream),
                    "dflash2_verify_reject");
}

// ------------------------------------------------------------------ Philox
int dflash2_philox4x64(const uint64_t* seed_dev, const int32_t* b, const int32_t* t, int n,
                       uint64_t* out, hipStream_t stream) {
  REQUIRE(n >= 0, DF2_ERR_SHAPE, "dflash2_philox4x64: n %d", n);
  if (n == 0) return DF2_OK;
  REQUIRE(seed_dev && b && t && out, DF2_ERR_NULL, "dflash2_philox4x64: null pointer argument");
  return hip_status(launch_philox(seed_dev, b, t, n, out, stream), "dflash2_philox4x64");
}

}  // extern "C"

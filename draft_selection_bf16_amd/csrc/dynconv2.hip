// dynconv2.hip -- two-tap dynamic depthwise convolution.
//
// "DFlash 2: Keep Drafting Parallel", section "A lightweight local
// convolution", equation Conv_k(x)_t = k_{t,0} (.) x_t + k_{t,1} (.) x_{t-1}:
// each tap is a learned base kernel plus a correction computed from the
// current hidden state, one correction per 16 channels; the first position
// reads the last verified token (Fig. 4).  With c_t = W x_t in R^{2G}:
//   y_t[ch] = (base0[ch] + c_t[ch/16]) x_t[ch] + (base1[ch] + c_t[G + ch/16]) x_{t-1}[ch].
//
// Two launches per application:
//  1. the tap corrections c = X W^T on the matrix cores (gemm.hip; M = B*L
//     rows, N = 2G, K = d: a skinny product), with the reduction over d
//     split into slices so that about one work-group per CU shares it; each
//     slice writes its own partial product;
//  2. a streaming epilogue, one work-group per (b, t) row: sums the slice
//     partials of its 2G taps in a fixed order into LDS and combines them
//     with x_t and x_{t-1} (16-byte loads, issued together with the partial
//     loads) into y (bf16 round-to-nearest-even, or fp32), written with
//     streaming stores (y is read by a later launch; measured: the batch-32
//     / block-16 step 0.4865 -> 0.4752 ms with these alone).  Its loads are
//     streaming loads too: cached ones fill the caches with lines that are
//     read at most twice (x_t, as the next row's x_{t-1}, is still found),
//     and the reads of the stages after the conv slow down (step 0.4565 ->
//     0.4464 ms; the projection 60.1 -> 57.3 us).
#include "df2_device.h"
#include "df2_internal.h"

namespace df2 {
namespace {

// Epilogue work-groups of 640 threads, one 16-byte chunk of x_t and of
// x_{t-1} each in flight (the whole row at d = 5120; a larger d loads its
// further chunks in the output loop).  Batch 32 / block 16 step (ms) and the
// stress cycle (us): 256 threads with three chunks each 0.4418 / 801; 320
// threads 0.4306 / 790; 512 0.4331 / 802; 640 with three chunk slots
// 0.4383 / 826 (their registers cost residency at 1,024 rows); 640 with one
// 0.4215 / 784.6.
constexpr int kThreads = 640;
constexpr int kMaxTaps = 2048;   // 2G <= 2048  <=>  d <= 16384
constexpr int kMaxSplit = 16;    // K slices of the tap GEMM
constexpr int kCUs = 256;        // MI355X

constexpr int kChunks = 1;       // 16-byte x chunks per thread requested before the first wait

// One work-group per (b, t) row.  Everything the row needs is requested
// before the first wait: the thread's x_t / x_{t-1} chunks, and, for
// threads < 2G/4, four taps' partial products of every slice (16-byte
// loads).  The taps are summed over the slices in a fixed order into LDS;
// after one barrier every thread writes its chunks of y.  Rows are spread so
// that consecutive rows run on one XCD (work-group i on XCD i mod 8), where
// x_{t-1} is the previous row's x_t, already in that XCD's L2.
template <bool Y_BF16>
// The arguments a work-group needs first (all but y) fit the 56 bytes that
// the command processor preloads into SGPRs, the grid size among them, so
// the kernel starts without a scalar load (y is fetched behind the loads).
__global__ __launch_bounds__(kThreads) void conv_epilogue_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ x_prev,
    const float* __restrict__ base, const float* __restrict__ part, int ksplit, int nb, int64_t kstride,
    int L, int d, void* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) float sc[kMaxTaps];
  const int full = nb / 8 * 8;
  const int bid = blockIdx.x;
  const int row = bid < full ? (bid % 8) * (full / 8) + bid / 8 : bid;   // b * L + t
  const int b = row / L, t = row % L;
  const int G = d / 16, NT = 2 * G, nch = d / 8;
  const int tid = threadIdx.x;
  const uint16_t* xt = x + (int64_t)row * d;
  const uint16_t* xp = t > 0 ? x + (int64_t)(row - 1) * d : (x_prev ? x_prev + (int64_t)b * d : nullptr);
  u32x4 vx[kChunks], vp[kChunks];
#pragma unroll
  for (int i = 0; i < kChunks; ++i) {
    const int c8 = tid + kThreads * i;
    const int cc = c8 < nch ? c8 : nch - 1;   // clamped: loaded, not used
    vx[i] = __builtin_nontemporal_load((const u32x4*)(xt + cc * 8));
    vp[i] = xp ? __builtin_nontemporal_load((const u32x4*)(xp + cc * 8)) : u32x4{0u, 0u, 0u, 0u};
  }
  for (int n4 = tid; n4 < NT / 4; n4 += kThreads) {
    const float* p = part + (int64_t)row * NT + n4 * 4;
    // slices in a fixed order, in blocks of 8 loads in flight (a slice past
    // ksplit reloads slice 0 and is not added)
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < ksplit; s0 += 8) {
      f32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[u] = __builtin_nontemporal_load((const f32x4*)(p + (int64_t)(s0 + u < ksplit ? s0 + u : 0) * kstride));
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (s0 + u < ksplit) acc += v[u];
    }
    *(f32x4*)(sc + n4 * 4) = acc;
  }
  __syncthreads();
  // 8 channels per 16-byte chunk; channel groups of 16 never straddle one
  for (int c8 = tid; c8 < nch; c8 += kThreads) {
    const int i = c8 / kThreads;   // the same for the whole work-group
    u32x4 ax = {0u, 0u, 0u, 0u}, ap = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int q = 0; q < kChunks; ++q)
      if (q == i) {
        ax = vx[q];
        ap = vp[q];
      }
    if (i >= kChunks) {
      ax = __builtin_nontemporal_load((const u32x4*)(xt + c8 * 8));
      ap = xp ? __builtin_nontemporal_load((const u32x4*)(xp + c8 * 8)) : u32x4{0u, 0u, 0u, 0u};
    }
    const int ch0 = c8 * 8, g = ch0 / 16;
    const float c0 = sc[g], c1 = sc[G + g];
    // base kernels: four 16-byte loads under one uniform branch
    f32x4 b0[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}}, b1[2] = {b0[0], b0[0]};
    if (base) {
      b0[0] = *(const f32x4*)(base + ch0);
      b0[1] = *(const f32x4*)(base + ch0 + 4);
      b1[0] = *(const f32x4*)(base + d + ch0);
      b1[1] = *(const f32x4*)(base + d + ch0 + 4);
    }
    float out[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t wx = ax[e >> 1], wp = ap[e >> 1];
      const float fx = (e & 1) ? bf16_hi(wx) : bf16_lo(wx);
      const float fp = (e & 1) ? bf16_hi(wp) : bf16_lo(wp);
      const float k0 = base ? b0[e >> 2][e & 3] + c0 : c0;
      const float k1 = base ? b1[e >> 2][e & 3] + c1 : c1;
      out[e] = fmaf(k0, fx, k1 * fp);
    }
    if (Y_BF16) {
      u32x4 o;
#pragma unroll
      for (int h = 0; h < 4; ++h)
        o[h] = (uint32_t)f32_to_bf16_rne(out[2 * h]) | ((uint32_t)f32_to_bf16_rne(out[2 * h + 1]) << 16);
      __builtin_nontemporal_store(o, (u32x4*)((uint16_t*)y + (int64_t)row * d + ch0));
    } else {
      float* yo = (float*)y + (int64_t)row * d + ch0;
      __builtin_nontemporal_store(f32x4{out[0], out[1], out[2], out[3]}, (f32x4*)yo);
      __builtin_nontemporal_store(f32x4{out[4], out[5], out[6], out[7]}, (f32x4*)(yo + 4));
    }
  }
}

}  // namespace

ConvPlan conv_plan(int B, int L, int d, int group) {
  (void)group;
  ConvPlan p;
  // 64 x 128 tiles in 4 LDS stages (96 KB) on eight waves in two
  // alternating groups (batch 32 / block 16 step 0.4455-0.4470 -> 0.4419-
  // 0.4422 ms against four waves over 3 stages; 3, 5 or 6 stages with the
  // eight waves 0.4606, 0.4498, 0.4555); from 1,024 rows on 128 x 128
  // tiles, which halve the W bytes per work-group (64 requests, block 16:
  // 926.4 against 949.1 us per cycle with 20 sites), on the same loop
  // (874 -> 861 us against four waves)
  const int M = B * L, N = 2 * (d / 16);
  p.tiling = M >= 1024 ? GemmTiling{128, 128, 4, 8, 3} : GemmTiling{64, 128, 4, 8, 3};
  const int bm = p.tiling.bm;
  const int tiles = ((M + bm - 1) / bm) * ((N + 127) / 128);
  const int nk = d / 64;
  // K slices: about one work-group per CU (one balanced round; two per CU
  // doubles the partial sums the epilogue reads), slices of >= 4 K-tiles and
  // at most kMaxSplit slices (the epilogue's limit).  Measured at M = 512,
  // d = 5120 in a replayed graph: 40 tiles x 6 slices 20.1 us per
  // application; 64 x 160 tiles x 8 slices, whose slices line up with the
  // XCDs (a quarter of the HBM fetch), 20.9 us: 1.3x the partial sums cost
  // more than the saved fetch.
  int ks = kCUs / (tiles > 0 ? tiles : 1);
  if (ks > nk / 4) ks = nk / 4;
  if (ks > kMaxSplit) ks = kMaxSplit;
  if (ks < 1) ks = 1;
  p.ksplit = ks;
  p.ws_bytes = align256((size_t)ks * (size_t)M * (size_t)N * sizeof(float));
  return p;
}

hipError_t launch_dynconv2(const void* x, const void* x_prev, const void* w, const float* base,
                           int B, int L, int d, int group, void* y, int y_dt, void* ws,
                           const ConvPlan& plan, hipStream_t stream) {
  (void)group;
  const int M = B * L, G = d / 16, N = 2 * G;
  if (M == 0) return hipSuccess;
  float* part = (float*)ws;
  GemmSeg s{};
  s.x = (const uint16_t*)x;
  s.gather = nullptr;
  s.x_rows = M;
  s.ldx = d;
  s.M = M;
  s.w0 = (const uint16_t*)w;
  s.w1 = (const uint16_t*)w;
  s.n0 = N;
  s.N = N;
  s.out = part;
  s.ldo = N;
  s.out_kstride = (int64_t)M * N;
  s.gate = 0;
  hipError_t e = launch_gemm(&s, 1, d, plan.ksplit, plan.tiling, "conv_gemm", stream);
  if (e != hipSuccess) return e;
  ProfileScope ps("conv_epilogue", stream);
  if (y_dt == 1)
    DF2_TRY(launch(conv_epilogue_kernel<true>, dim3(M), dim3(kThreads), 0, stream, ps,
        (const uint16_t*)x, (const uint16_t*)x_prev, base, part, plan.ksplit, M, (int64_t)M * N, L, d, y));
  else
    DF2_TRY(launch(conv_epilogue_kernel<false>, dim3(M), dim3(kThreads), 0, stream, ps,
        (const uint16_t*)x, (const uint16_t*)x_prev, base, part, plan.ksplit, M, (int64_t)M * N, L, d, y));
  return hipGetLastError();
}

// ---------------------------------------------------------------- Philox words
namespace {
__global__ void philox_kernel(const uint64_t* __restrict__ seed_dev, const int32_t* __restrict__ b,
                              const int32_t* __restrict__ t, int n, uint64_t* __restrict__ out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  u64x4 o = philox4x64_10(seed_dev[0], 0, (uint64_t)(uint32_t)t[i], (uint64_t)(uint32_t)b[i], 0, 0);
#pragma unroll
  for (int k = 0; k < 4; ++k) out[(int64_t)i * 4 + k] = o.w[k];
}
}  // namespace

hipError_t launch_philox(const uint64_t* seed_dev, const int32_t* b, const int32_t* t, int n,
                         uint64_t* out, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  ProfileScope ps("philox", stream);
  DF2_TRY(launch(philox_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, ps, seed_dev, b, t, n, out));
  return hipGetLastError();
}

}  // namespace df2

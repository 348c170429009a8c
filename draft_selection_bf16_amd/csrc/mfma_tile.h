// mfma_tile.h -- pieces shared by the bf16 MFMA kernels that stage K-tiles
// of two K-contiguous operands through LDS (gemm.hip, lmhead.hip).
// Internal; not part of the ABI.
//
// LDS stage = X tile [BM][64] then W tile [BN][64], rows of 128 bytes.  One
// direct buffer-to-LDS load instruction of a wave fills 1 KB = 8 rows: lane
// i writes the 16-byte slot (row i / 8, slot i % 8) and fetches the chunk
// slot ^ swz(row) of that row, so the 16-byte chunks of a row are stored in
// swizzled order.  With chunk c of row r stored at c ^ (r mod 8), the MFMA
// fragment reads (16 consecutive rows, one chunk each) are free of bank
// conflicts: 4 LDS cycles per 16-byte read of a wave, measured with the
// bank-conflict counter (an extra ^ (r / 8 mod 2) term doubles it to 8).
// Rows outside the problem get an out-of-range lane offset: the hardware
// writes zeros for them.
#pragma once

#include "df2_device.h"

namespace df2 {
namespace mfma {

constexpr int BK = 64;   // K-tile width (bf16 elements: one 128-byte row)

__device__ __forceinline__ int swz(int r) { return r & 7; }

// One direct buffer-to-LDS load of 16 bytes per lane (a plain device
// function: called from a kernel template directly, the builtin keeps the
// host-side launch stub from being emitted).
typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, soff, 0, 0);
}

// s_waitcnt immediate that waits until at most n vector-memory operations
// of this wave are outstanding (expcnt and lgkmcnt left unconstrained)
__host__ __device__ constexpr int vmcnt_imm(int n) {
  return (n & 15) | (7 << 4) | (15 << 8) | (((n >> 4) & 3) << 14);
}

// The K loop of a tile of FM x FN 16 x 16 blocks per wave with the eight
// waves in two alternating groups of four (group g holds the waves of tile
// rows g BM / 2 .. (g + 1) BM / 2 - 1, one wave of each group per SIMD).
// Every K-tile takes two phases, with a
// work-group barrier after each: in its memory phase a group reads all its
// fragments of tile t from LDS and issues its copies of tile t + S - 1; in
// its compute phase it runs the MFMAs on them.  Group 1 starts one phase
// late, so in every phase one wave of each SIMD feeds the matrix pipe while
// the other reads LDS -- with both groups in step, each SIMD's two waves
// read at the same time and then wait on the matrix pipe together.
// Ordering: a group's fragment reads of tile t are complete (lgkmcnt) and its
// copies of tile t + 1 have landed (vmcnt) before the barrier that ends its
// memory phase, which precedes every read of tile t + 1; the stage of tile
// t - 1 that a memory phase's copies overwrite was read (completely) one and
// two phases earlier.  Summation order per accumulator is the
// same as in the single-group loop (K-tiles in order, two K steps each).
// Measured: the batch-32 projection 49.3 -> 47.6 us; the fused LM heads
// (lmhead.hip) 2 % faster with 256-row tiles, unchanged with 128-row ones
// (1,071 us either way), which keep the single-group loop.
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// lds: the stages (tile t in stage t % S, STAGE bytes each); issue(t):
// this wave's copies of tile t (LPW load instructions, empty past the
// end); ao / bo: the lane's fragment offsets in a stage for the two K
// steps; the S - 1 first tiles are already issued.
template <int S, int FM, int FN, int LPW, int STAGE, typename Issue>
__device__ __forceinline__ void pingpong_loop(const uint8_t* lds, Issue& issue, const int (&ao)[FM][2],
                                              const int (&bo)[FN][2], f32x4 (&acc)[FM][FN], int nk, int grp) {
  static_assert(S >= 3, "tile t + 1 in flight while tile t is read");
  // vmcnt: tiles t + 2 .. t + S - 1 may still be in flight; lgkmcnt: 0
  constexpr int kWait = ((S - 2) * LPW & 15) | (7 << 4) | ((((S - 2) * LPW) >> 4) & 3) << 14;
  __builtin_amdgcn_s_waitcnt(vmcnt_imm((S - 2) * LPW));   // this wave's copies of tile 0
  phase_barrier();
  if (grp == 1) phase_barrier();
  for (int t = 0; t < nk; ++t) {
    const uint8_t* st = lds + (t % S) * STAGE;
    bf16x8 a[2][FM], b[2][FN];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
      for (int i = 0; i < FM; ++i) a[s2][i] = *(const bf16x8*)(st + ao[i][s2]);
#pragma unroll
      for (int j = 0; j < FN; ++j) b[s2][j] = *(const bf16x8*)(st + bo[j][s2]);
    }
    issue(t + S - 1);
    __builtin_amdgcn_s_waitcnt(kWait);
    phase_barrier();
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s2][i], b[s2][j], acc[i][j], 0, 0, 0);
    phase_barrier();
  }
  if (grp == 0) phase_barrier();
}

}  // namespace mfma
}  // namespace df2

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

}  // namespace mfma
}  // namespace df2

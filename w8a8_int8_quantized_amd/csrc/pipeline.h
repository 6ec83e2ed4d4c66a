// Global -> LDS staging shared by the large-M GEMM kernels (gfx950).
//
// Operand tiles stream through LDS in K blocks of 128 bytes per row (one
// 128-byte cache line per row), filled by direct-to-LDS buffer loads
// ("buffer_load_dwordx4 ... lds": no staging registers, no ds_write).  One
// such load moves 8 rows x 128 bytes; lane i lands in 16-byte slot i of a
// 1 KB block, so the block holds rows r..r+7 row-major.  The lane->address map
// applies an XOR swizzle for free: lane i fetches chunk (i & 7) ^ (row & 7),
// i.e. 16-byte chunk c of row r is stored at position c ^ (r & 7).  An MFMA
// fragment read (16 or 32 consecutive rows, one chunk each) then touches 8
// distinct bank groups per 8 lanes: no LDS bank conflicts.
//
// The buffer descriptor bounds every load to the operand tile's valid rows:
// rows past the end of A or W read as zero, so ragged tiles need no clamping.
#pragma once

#include "common.h"

namespace w8 {

typedef int v16i __attribute__((ext_vector_type(16)));

// s_waitcnt with explicit counters (vmcnt split over bits [3:0] and [15:14],
// expcnt [6:4] left at its maximum, lgkmcnt [11:8]).
template <int VM, int LGKM>
__device__ __forceinline__ void waitcnt() {
  constexpr int e = (VM & 15) | (7 << 4) | ((LGKM & 15) << 8) | ((VM >> 4) << 14);
  __builtin_amdgcn_s_waitcnt(e);
}

// Workgroup barrier that the compiler may not move memory accesses across.
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

// s_waitcnt and s_barrier as one statement with a memory clobber: the
// scheduler can move no LDS read of this wave below the wait (the
// s_waitcnt builtin alone does not order memory accesses), so every read
// issued before it has completed when the barrier releases the other waves.
template <int VM, int LGKM>
__device__ __forceinline__ void wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(%1)\n\ts_barrier" ::"n"(VM), "n"(LGKM) : "memory");
}

// Raw buffer descriptor: base, no stride, `bytes` valid bytes.
__device__ __forceinline__ v4i make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  v4i r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32) & 0xffff);
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000;
  return r;
}

// 16 bytes per lane from (voff + soff) into LDS at lds + 16 * lane.  The load
// has no register result, so nothing can be overwritten while it is in
// flight; completion is tracked with vmcnt by the caller.
__device__ __forceinline__ void dma16(v4i rsrc, int voff, int soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               ::"s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
               : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)p;
}

// Per-lane offset of this lane's 16 bytes inside a DMA block: row (lane >> 3)
// of the block, swizzled chunk.
__device__ __forceinline__ int dma_lane_off(int lane, int K) {
  return (lane >> 3) * K + (((lane & 7) ^ (lane >> 3)) << 4);
}

// LDS byte offset (inside a tile) of the 16 bytes a lane reads for an MFMA
// fragment: row (lane % rows_per_frag) of the fragment's row group, chunk c.
__device__ __forceinline__ int frag_off(int row_in_group, int chunk) {
  return row_in_group * 128 + ((chunk ^ (row_in_group & 7)) << 4);
}

}  // namespace w8

// tile_layout.hpp - swizzled row-major LDS tiles shared by the attention
// kernels: 16-byte chunk placement for tiles filled by LDS-direct loads and
// read with ds_read_b128 (16 rows at one chunk) and ds_read_b64_tr_b16
// (4 rows x 32 bytes), plus the wait helper for those loads.
#pragma once

#include "device_common.hpp"

namespace attn97 {

// Block order.  Workgroups are dispatched to the eight XCDs in turn (block
// id mod 8) and, within an XCD, in id order.  grouped (and BH a multiple of
// 8): block id takes head x + 8 (s / n) and tile s mod n (x = id mod 8,
// s = id / 8): each XCD owns whole heads and runs one head's n tiles one
// after another, so the workgroups an XCD runs together stream the same
// head's operand tiles through its L2.  Otherwise head id mod BH, tile
// id / BH: tile t of every head before tile t + 1 of any (with B*H a
// multiple of 8 each head still on one XCD), the order that puts a causal
// pass's heaviest tiles first across the whole grid.  n: tiles per head
// (gridDim.x / BH).
__device__ __forceinline__ void xcd_head_order(int id, int BH, int n, bool grouped, int& bh, int& t) {
  if (grouped && BH % 8 == 0) {
    const int x = id & 7, s = id >> 3;
    bh = x + 8 * (s / n);
    t = s - (s / n) * n;
  } else {
    bh = id % BH;
    t = id / BH;
  }
}

// Physical 16-byte chunk index, inside a K or V tile, of logical chunk c of
// row `row`.  Rows of 256 bytes (D = 128) or 512 bytes (D = 256) XOR the low
// four bits of the chunk with f(row) = ((row & 3) << 2) | ((row >> 2) & 3),
// which is distinct over 16 consecutive rows and moves each group of four
// consecutive rows to distinct 64-byte quarters.  Rows of 128 bytes (D = 64)
// pair up into 256-byte lines and XOR the chunk-in-line with
// g(line) = ((line & 1) << 2) | ((line >> 1) & 3).
template <int D>
__device__ __forceinline__ int swz_chunk(int row, int c) {
  if constexpr (D == 64) {
    const int line = row >> 1;
    const int cl = ((row & 1) << 3) | c;
    const int g = ((line & 1) << 2) | ((line >> 1) & 3);
    return (line << 4) | (cl ^ g);
  } else {
    const int f = ((row & 3) << 2) | ((row >> 2) & 3);
    return row * (D / 8) + (c ^ f);
  }
}

// Inverse: logical (row, chunk) stored at physical chunk P.
template <int D>
__device__ __forceinline__ void unswz_chunk(int P, int& row, int& c) {
  if constexpr (D == 64) {
    const int line = P >> 4;
    const int g = ((line & 1) << 2) | ((line >> 1) & 3);
    const int cl = (P & 15) ^ g;
    row = 2 * line + (cl >> 3);
    c = cl & 7;
  } else {
    row = P / (D / 8);
    const int f = ((row & 3) << 2) | ((row >> 2) & 3);
    c = (P % (D / 8)) ^ f;
  }
}

// Word 3 of a raw buffer resource (stride 0, 32-bit data format, no
// thread-id swizzle), as used for the gfx9-family buffer instructions.
constexpr int kBufRsrcWord3 = 0x00020000;

// Copy BYTES (16 or 4) per lane from global memory straight into LDS: lane l
// reads base + voff (bytes) and writes lds + BYTES * l (lds is wave-uniform).
// It is a buffer load with the LDS bit over the resource [base, base +
// extent), not the FLAT-encoded global_load_lds.  With a FLAT LDS load in
// flight the compiler has to assume it may complete out of order on the LDS
// counter and makes every later LDS read wait for all outstanding ones
// (lgkmcnt(0)); buffer loads count on the vector-memory counter only, so the
// MFMA operand reads keep exact partial waits and stay ahead of the MFMAs.
// Offsets at or past `extent` read zero.
// base and extent must be the same in every lane of the wavefront; they are
// read from the first active lane (a resource the compiler cannot prove
// uniform would otherwise become a loop over the distinct values).
template <int BYTES>
__device__ __forceinline__ void lds_dma(const void* base, uint32_t extent, uint32_t voff, void* lds) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  void* ub = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  const int ue = __builtin_amdgcn_readfirstlane((int)extent);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, ue, kBufRsrcWord3);
  static_assert(BYTES == 16 || BYTES == 4, "16 or 4 bytes per lane");
  if constexpr (BYTES == 16)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 4, voff, 0, 0, 0);
}

// s_waitcnt with vmcnt <= N, lgkmcnt = 0, expcnt unconstrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm_lds() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
}

// Workgroup barrier that does not drain outstanding global->LDS loads.
// __syncthreads() waits for every outstanding memory operation first, which
// would forbid keeping tile loads in flight across a barrier; the callers
// wait explicitly (wait_vm_lds) for exactly the loads they need.  The memory
// clobber keeps the compiler from moving LDS accesses across the barrier.
__device__ __forceinline__ void barrier_keep_loads() { asm volatile("s_barrier" ::: "memory"); }

// Distinct empty asm at the top of the masked and the unmasked variant of a
// tile step.  Both variants begin with the same LDS operand reads; without a
// differing first instruction the compiler merges those reads into the block
// before the branch, outside the reach of the step's read-ahead schedule,
// and holds every fragment of the tile in registers at once.
template <bool MASK>
__device__ __forceinline__ void tile_marker() {
  if constexpr (MASK)
    asm volatile("; masked tile" ::: "memory");
  else
    asm volatile("; interior tile" ::: "memory");
}

}  // namespace attn97

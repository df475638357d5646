// tile_layout.hpp - swizzled row-major LDS tiles shared by the attention
// kernels: 16-byte chunk placement for tiles filled by global_load_lds and
// read with ds_read_b128 (16 rows at one chunk) and ds_read_b64_tr_b16
// (4 rows x 32 bytes), plus the wait helper for those loads.
#pragma once

#include "device_common.hpp"

namespace attn97 {

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

// device_common.hpp - types and small device helpers shared by the gfx950
// attention kernels: the bf16 MFMA wrapper, LDS fragment loads, the two
// exp2 implementations and the tile-transposing LDS store.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_kernels.hpp"

namespace attn97 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// ---------------------------------------------------------------------------
// MFMA.  v_mfma_f32_32x32x16_bf16 computes D = A*B + C for a 32x32 output
// tile with a 16-deep reduction.  Lane l (h = l/32, c = l%32) supplies
//   A[row c][k = 8h .. 8h+7]   and   B[k = 8h .. 8h+7][col c]
// and holds the output column c, rows 8*(r/4) + 4h + (r%4) for r = 0..15.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// 16-byte LDS read (ds_read_b128); p must be 16-byte aligned.
__device__ __forceinline__ bf16x8 lds_frag(const uint16_t* p) {
  return as_bf16x8(*reinterpret_cast<const u32x4*>(p));
}

// Round eight fp32 values to bf16 (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16x8 to_bf16x8(float a0, float a1, float a2, float a3, float a4,
                                            float a5, float a6, float a7) {
  f32x8 v = {a0, a1, a2, a3, a4, a5, a6, a7};
  return __builtin_convertvector(v, bf16x8);
}

__device__ __forceinline__ u32x2 pack_bf16x4(float a0, float a1, float a2, float a3) {
  f32x4 v = {a0, a1, a2, a3};
  return __builtin_bit_cast(u32x2, __builtin_convertvector(v, bf16x4));
}

// ---------------------------------------------------------------------------
// Key (or query) order inside a 16-wide group when a tile is stored
// transposed in LDS.  The scores of a 32x32 MFMA tile leave lane half h with
// rows {8a + 4h + e : a = 0,1; e = 0..3} of each 16-row group.  Storing row
// 16t + 8a + 4h + e at position 16t + 8h + 4a + e makes those eight rows one
// contiguous 16-byte run, so the matching operand of the next MFMA is a
// single ds_read_b128.  `g` is the index of a group of four rows.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int perm_pos_of_group(int g) {
  return 16 * (g >> 2) + 8 * (g & 1) + 4 * ((g >> 1) & 1);
}
__device__ __forceinline__ int perm_pos_of_row(int r) {
  return perm_pos_of_group(r >> 2) + (r & 3);
}

// Store a 4-row x 8-column bf16 block (rows[i] = row i, eight columns) into a
// transposed LDS tile dst[col][pos .. pos+3] (column-major rows, stride rs).
__device__ __forceinline__ void store_transposed_4x8(uint16_t* dst, int rs, int col0, int pos,
                                                     const u32x4 rows[4]) {
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    uint32_t a0 = rows[0][m], a1 = rows[1][m], a2 = rows[2][m], a3 = rows[3][m];
    u32x2 lo = {(a0 & 0xffffu) | (a1 << 16), (a2 & 0xffffu) | (a3 << 16)};
    u32x2 hi = {(a0 >> 16) | (a1 & 0xffff0000u), (a2 >> 16) | (a3 & 0xffff0000u)};
    *reinterpret_cast<u32x2*>(dst + (col0 + 2 * m) * rs + pos) = lo;
    *reinterpret_cast<u32x2*>(dst + (col0 + 2 * m + 1) * rs + pos) = hi;
  }
}

// ---------------------------------------------------------------------------
// exp2.  Native: the hardware transcendental v_exp_f32.  Poly: the software
// exponential on the fused multiply-add pipe (the pages' FA-4 technique):
// x = n + f with n = floor(x), f in [0,1); 2^f by a degree-3 polynomial with
// p(0) = 1 fitted for minimum relative error (max 8.6e-5, fit_exp2.py);
// 2^n applied by v_ldexp_f32.  x is clamped at -127.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float exp2_native(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float exp2_poly(float x) {
  x = __builtin_fmaxf(x, -127.0f);
  float fl = __builtin_floorf(x);
  float f = x - fl;
  int n = (int)fl;
  float p = __builtin_fmaf(7.706803083e-02f, f, 2.276435345e-01f);
  p = __builtin_fmaf(p, f, 6.951172948e-01f);
  p = __builtin_fmaf(p, f, 1.0f);
  return __builtin_amdgcn_ldexpf(p, n);
}

// Kernel exp2 modes (kExpNative, kExpPoly, exp_mix(q), attn_kernels.hpp):
// in the mixed modes the polynomial takes q of every four elements (element
// idx with idx % 4 < q) and the native unit the rest.
template <int MODE>
__device__ __forceinline__ float exp2_mode(float x, int idx) {
  if constexpr (MODE == kExpNative) {
    return exp2_native(x);
  } else if constexpr (MODE == kExpPoly) {
    return exp2_poly(x);
  } else {
    constexpr int q = MODE - 1;
    static_assert(q >= 1 && q <= 3, "mixed mode: one to three of every four elements polynomial");
    return ((idx & 3) < q) ? exp2_poly(x) : exp2_native(x);
  }
}

// The value of lane l ^ 32.  v_permlane32_swap (gfx950) called with one
// register as both operands returns [0]: the lower half's values in the
// upper lanes, [1]: the upper half's values in the lower lanes; no LDS round
// trip, unlike a general shuffle.
__device__ __forceinline__ float wave_swap_halves(float x) {
  const unsigned int u = __builtin_bit_cast(unsigned int, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (threadIdx.x & 32) ? r[0] : r[1]);
}

}  // namespace attn97

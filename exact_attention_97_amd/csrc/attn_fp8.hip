// attn_fp8.hip - FP8 (OCP E4M3) forward attention with incoherent processing,
// D = 128.
//
// Page "FlashAttention-3 и FlashAttention-4", section "Поддержка FP8 с
// контролем ошибок": before the rounding to FP8, Q and K pass through a
// cheap transform that spreads outliers over the coordinates.  Here the
// transform is x -> (x * s) H / sqrt(D) with H the Sylvester-Hadamard matrix
// and s caller-given random signs; it is orthogonal, so Q K^T is unchanged.
//
// Two steps:
//  * quantize: Q and K rows transformed (a 128-point fast Walsh-Hadamard
//    transform in float64 registers, one row per four lanes) and rounded to
//    E4M3 with one scale per Q row and one per (batch, head) for K (a pass
//    over the transformed K finds the head's maximum first); V rounded with
//    one scale per column (a column-maximum kernel runs first) and stored
//    transposed, keys permuted inside each 64-key group so that the PV
//    operand of a lane is 32 contiguous bytes.  Every code is the rounding
//    of the float64 quotient x * 448 / max|x|, straight to E4M3.
//  * forward: the online-softmax kernel of the bf16 path with both products
//    on v_mfma_f32_32x32x64_f8f6f4 (twice the bf16 MFMA rate): S^T = K Q^T
//    and O^T += V^T P^T with P rounded to E4M3 in registers.  The product
//    contracts lane half h and byte j of both operands against each other,
//    so any assignment of the 64 contraction indices to (h, j) works as long
//    as both operands use it: K and Q use d = 64 t + 32 h + j, P and V^T use
//    the key order in which the score MFMA leaves P in its accumulators.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "attn_kernels.hpp"
#include "device_common.hpp"
#include "tile_layout.hpp"

namespace attn97 {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int FD = 128;   // head dim
constexpr int FBC = 64;   // keys per tile
constexpr int FBR = 128;  // query padding of the buffer (rows per four-wavefront workgroup)
constexpr float kE4M3Max = 448.0f;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// y (|y| <= 448) rounded to the nearest E4M3 value, ties to even, straight
// from float64 (no intermediate float32 rounding, which could land a value
// near a midpoint exactly on it).  E4M3 values are multiples of 2^(E - 3) in
// the binade [2^E, 2^(E+1)) for E >= -6, and of 2^-9 below 2^-6, so the
// value is rint(|y| / q) q with q that quantum (a power of two: both scalings
// are exact).  The result is exactly representable in float32 and in E4M3;
// its sign is y's (a negative value that rounds to zero keeps the sign).
__device__ __forceinline__ float round_e4m3_f64(double y) {
  const double a = __builtin_fabs(y);
  const int e = __builtin_amdgcn_frexp_exp(a);  // a = f 2^e, f in [0.5, 1): E = e - 1
  const int q = (e - 1 > -6 ? e - 1 : -6) - 3;
  const float r = (float)__builtin_ldexp(__builtin_rint(__builtin_ldexp(a, -q)), q);
  return y < 0.0 ? -r : r;
}

// E4M3 code of x relative to a group maximum amax > 0: x * 448 / amax as a
// float64 quotient (x * 448 is exact for the inputs here; the division is
// IEEE, correctly rounded), rounded straight to E4M3.  amax = 0: code 0.
__device__ __forceinline__ float e4m3_value_of(double x, double amax) {
  return amax > 0.0 ? round_e4m3_f64((x * (double)kE4M3Max) / amax) : 0.0f;
}

// four floats to four E4M3 bytes (round to nearest even), byte i = x_i
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  // format codes 0 / 0: both operands E4M3; no block scales
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ i32x8 lds_frag32(const uint8_t* p0, const uint8_t* p1) {
  const u32x4 a = *reinterpret_cast<const u32x4*>(p0);
  const u32x4 b = *reinterpret_cast<const u32x4*>(p1);
  return i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
}

// The value of lane l ^ 32 (M = 32) or l ^ 16 (M = 16), by the gfx950
// half-swap instructions (no LDS round trip).  Called with the same register
// as both operands, v_permlane32_swap returns [0]: the lower 32 lanes' values
// in the upper lanes (own values below), [1]: the upper lanes' values in the
// lower lanes; v_permlane16_swap does the same between the 16-lane rows
// (0, 1) and (2, 3).  The partner's value is [0] in the upper lanes, [1] below.
template <int M>
__device__ __forceinline__ double lane_xor_f64(double x, bool upper) {
  typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
  const u32x2_t w = __builtin_bit_cast(u32x2_t, x);
  u32x2_t o;
  if constexpr (M == 32) {
    const auto a = __builtin_amdgcn_permlane32_swap(w[0], w[0], false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(w[1], w[1], false, false);
    o = upper ? u32x2_t{a[0], b[0]} : u32x2_t{a[1], b[1]};
  } else {
    static_assert(M == 16, "half or row swap");
    const auto a = __builtin_amdgcn_permlane16_swap(w[0], w[0], false, false);
    const auto b = __builtin_amdgcn_permlane16_swap(w[1], w[1], false, false);
    o = upper ? u32x2_t{a[0], b[0]} : u32x2_t{a[1], b[1]};
  }
  return __builtin_bit_cast(double, o);
}

// ---------------------------------------------------------------------------
// Transform and quantize Q and K.  Grid (Sp / 64, B*H, NZ), four wavefronts
// of 16 rows; lane l handles quarter qd = l >> 4 (elements 32 qd .. 32 qd +
// 31) of row l & 15.  Rows past S are zero (Q scale 1).
//
// PASS 0 (NZ = 1, K only): the maximum of |transformed K| of each head, by a
// workgroup reduction and one 64-bit atomic maximum per workgroup into the
// scratch region (non-negative doubles order like their bit patterns).
// PASS 1 (NZ = 2; z = 0 Q, z = 1 K): codes and scales; Q rows against their
// own maximum, K rows against their head's maximum from pass 0.
//
// The transform runs in float64: its outputs are sums of 128 bf16 values
// with signs, which float64 holds exactly (float32 would round them once
// outliers widen the range of the summands), so the codes depend on the
// exact transform only.  Its butterfly stages commute; the two across
// quarters are exchanges between lanes (H_2n x = [H_n (a + b); H_n (a - b)]
// for x = [a; b]), the other five run inside each lane.
// ---------------------------------------------------------------------------
template <int PASS>
__global__ __launch_bounds__(256) void fp8_qk_quant_kernel(const uint16_t* __restrict__ Q,
                                                           const uint16_t* __restrict__ K,
                                                           const float* __restrict__ signs, Fp8Buf f, int S) {
  __shared__ double wave_max[4];
  const int which = PASS == 0 ? 1 : blockIdx.z;
  const int bh = blockIdx.y;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int qd = lane >> 4;
  const int row = blockIdx.x * 64 + 16 * wave + (lane & 15);
  const int Sp = f.Sp;
  const uint16_t* src = (which ? K : Q) + (size_t)bh * S * FD;

  double x[32];
  if (row < S) {
    const u32x4* p = reinterpret_cast<const u32x4*>(src + (size_t)row * FD + 32 * qd);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const u32x4 w = p[c];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[8 * c + 2 * e] = (double)bf16_lo(w[e]);
        x[8 * c + 2 * e + 1] = (double)bf16_hi(w[e]);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = 0.0;
  }

  double norm = 1.0;
  if (signs != nullptr) {
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] *= (double)signs[32 * qd + i];
    // stage 64 (partner quarter qd ^ 2), then stage 32 (partner qd ^ 1): the
    // lane holding the upper part keeps (other - own), the lower one (own + other)
    {
      const bool upper = (lane & 32) != 0;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const double other = lane_xor_f64<32>(x[i], upper);
        x[i] = upper ? (other - x[i]) : (x[i] + other);
      }
    }
    {
      const bool upper = (lane & 16) != 0;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const double other = lane_xor_f64<16>(x[i], upper);
        x[i] = upper ? (other - x[i]) : (x[i] + other);
      }
    }
#pragma unroll
    for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        if ((i & h) == 0) {
          const double a = x[i], b = x[i + h];
          x[i] = a + b;
          x[i + h] = a - b;
        }
      }
    }
    norm = 0.088388347648318440550;  // 1 / sqrt(128)
  }

  double amax = 0.0;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = __builtin_fmax(amax, __builtin_fabs(x[i]));
  amax = __builtin_fmax(amax, __shfl_xor(amax, 16));  // the row's four quarters
  amax = __builtin_fmax(amax, __shfl_xor(amax, 32));
  double* kmax = reinterpret_cast<double*>(f.kmax);
  if constexpr (PASS == 0) {  // K: this workgroup's 64 rows, then the head
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) amax = __builtin_fmax(amax, __shfl_xor(amax, o));
    if (lane == 0) wave_max[wave] = amax;
    __syncthreads();
    if (tid == 0) {
      const double m = __builtin_fmax(__builtin_fmax(wave_max[0], wave_max[1]), __builtin_fmax(wave_max[2], wave_max[3]));
      atomicMax(reinterpret_cast<unsigned long long*>(kmax + bh), __builtin_bit_cast(unsigned long long, m));
    }
    return;
  } else {
    if (which == 1) amax = kmax[bh];  // the head's maximum
    // the transformed row is x * norm; its scale is max|x * norm| / 448 and
    // its codes are E4M3(x * norm / scale) = E4M3(x * 448 / max|x|), in which
    // the factor norm cancels
    const float sc = amax > 0.0 ? (float)(amax * norm / (double)kE4M3Max) : 1.0f;
    uint8_t* dst = (which ? f.k8 : f.q8) + ((size_t)bh * Sp + row) * FD + 32 * qd;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d = 16 * c + 4 * e;
        w[e] = pack_e4m3x4(e4m3_value_of(x[d], amax), e4m3_value_of(x[d + 1], amax), e4m3_value_of(x[d + 2], amax),
                           e4m3_value_of(x[d + 3], amax));
      }
      *reinterpret_cast<u32x4*>(dst + 16 * c) = w;
    }
    if (which == 0) {
      if (qd == 0) f.qs[(size_t)bh * Sp + row] = sc;
    } else if (blockIdx.x == 0 && tid == 0) {
      f.ks[bh] = sc;
    }
  }
}

// The scratch maxima start at zero: V's column maxima and K's head maxima.
__global__ __launch_bounds__(256) void fp8_clear_kernel(Fp8Buf f, int BH) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < BH * FD) f.vpart[i] = 0.0f;
  if (i < BH) reinterpret_cast<double*>(f.kmax)[i] = 0.0;
}

// Column maxima of V.  Grid (Sp / 128, B*H), 256 threads: thread t reads
// the 16-byte chunk t % 16 (columns 8 (t % 16) .. + 7) of rows t / 16 + 16 i
// of the 128-row chunk; the 16 row groups reduce through LDS, and each
// column's maximum goes into the scratch region with an integer atomicMax
// (non-negative floats order like their bit patterns).  fp8_clear_kernel,
// launched before on the same stream, zeroed those maxima.
__global__ __launch_bounds__(256) void fp8_v_amax_kernel(const uint16_t* __restrict__ V, Fp8Buf f, int S) {
  __shared__ float part[16][FD];
  const int chunk = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
  const int c = t & 15, rg = t >> 4;
  const uint16_t* src = V + (size_t)bh * S * FD + 8 * c;
  float m[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) m[j] = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = chunk * 128 + rg + 16 * i;
    if (r < S) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(src + (size_t)r * FD);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        m[2 * e] = __builtin_fmaxf(m[2 * e], __builtin_fabsf(bf16_lo(w[e])));
        m[2 * e + 1] = __builtin_fmaxf(m[2 * e + 1], __builtin_fabsf(bf16_hi(w[e])));
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) part[rg][8 * c + j] = m[j];
  __syncthreads();
  if (t < FD) {
    float mm = 0.0f;
#pragma unroll
    for (int g = 0; g < 16; ++g) mm = __builtin_fmaxf(mm, part[g][t]);
    atomicMax(reinterpret_cast<unsigned int*>(f.vpart) + (size_t)bh * FD + t, __builtin_bit_cast(unsigned int, mm));
  }
}

// V to E4M3, transposed: row d of head bh holds the Sp keys, and inside each
// 64-key group key 32 kb + 8 r4 + 4 h + e sits at byte 32 h + 16 kb + 4 r4 + e
// (h, kb in {0, 1}; r4, e in 0..3).  Grid (Sp / 64, B*H), 256 threads: the
// 64 x 128 tile comes in with coalesced 16-byte loads through LDS; thread
// (d, kb) then rounds keys 32 kb .. 32 kb + 31 of column d.  The first tile's
// workgroup also writes the column scales.
__global__ __launch_bounds__(256) void fp8_v_quant_kernel(const uint16_t* __restrict__ V, Fp8Buf f, int S) {
  __shared__ __attribute__((aligned(16))) uint16_t tv[FBC][FD];
  const int tile = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
  const int k0 = tile * FBC;
  const uint16_t* src = V + (size_t)bh * S * FD;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = t + 256 * i, row = idx >> 4, ch = idx & 15;
    const int key = k0 + row;
    const u32x4 w = key < S ? *reinterpret_cast<const u32x4*>(src + (size_t)key * FD + 8 * ch) : u32x4{0, 0, 0, 0};
    *reinterpret_cast<u32x4*>(&tv[row][8 * ch]) = w;
  }
  __syncthreads();
  const int d = t & 127, kb = t >> 7;
  const float m = __builtin_bit_cast(float, reinterpret_cast<const unsigned int*>(f.vpart)[(size_t)bh * FD + d]);
  if (tile == 0 && kb == 0) f.vs[(size_t)bh * FD + d] = m > 0.0f ? m / kE4M3Max : 1.0f;
  // v * 448 / m as in the Q / K quantizer: float64 quotient, rounded
  // straight to E4M3
  const double md = (double)m;
  u32x4 w[2];  // [h]: words r4 = 0..3
#pragma unroll
  for (int g8 = 0; g8 < 8; ++g8) {  // key group g = 8 kb + g8: keys 4 g .. 4 g + 3
    const int h = g8 & 1, r4 = g8 >> 1, key0 = 32 * kb + 4 * g8;
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = e4m3_value_of((double)bf16_lo((uint32_t)tv[key0 + e][d]), md);
    w[h][r4] = pack_e4m3x4(v[0], v[1], v[2], v[3]);
  }
  uint8_t* dst = f.v8t + ((size_t)bh * FD + d) * f.Sp + k0;
  *reinterpret_cast<u32x4*>(dst + 16 * kb) = w[0];
  *reinterpret_cast<u32x4*>(dst + 32 + 16 * kb) = w[1];
}

// ---------------------------------------------------------------------------
// Forward.  One workgroup of four wavefronts per 128 queries of one head;
// 64-key tiles of K (64 rows x 128 B) and V^T (128 rows x 64 B) stream
// through two LDS buffers each with LDS-direct buffer loads.  16-byte chunks are
// XOR-swizzled (K: chunk ^ ((key >> 1) & 7); V^T: chunk ^ ((d >> 2) & 3)) so
// that each 16-lane group of a 128-bit operand read hits 16 distinct bank
// groups.
// ---------------------------------------------------------------------------
struct Fp8Wave {
  // LDS byte offsets of this lane's operand chunks (block 0 / d-block 0)
  int kfrag[2][2];  // [t][half]: key row c32, chunks 4 t + 2 hh + half
  int vfrag[2];     // [half]: row c32 of V^T, chunks 2 hh + half
  uint32_t kdma[2], vdma[2];  // DMA source offsets (bytes) of this lane's chunks

  // NCH = 16-byte chunks per lane of one 8 KiB tile (2 with four
  // wavefronts, 1 with eight)
  template <int NCH>
  __device__ __forceinline__ void init(int wave, int lane, int Sp) {
    const int hh = lane >> 5, c32 = lane & 31;
    const int kx = (c32 >> 1) & 7, vx = (c32 >> 2) & 3;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int h = 0; h < 2; ++h) kfrag[t][h] = c32 * FD + (((4 * t + 2 * hh + h) ^ kx) * 16);
#pragma unroll
    for (int h = 0; h < 2; ++h) vfrag[h] = c32 * FBC + (((2 * hh + h) ^ vx) * 16);
#pragma unroll
    for (int n = 0; n < NCH; ++n) {
      const int P = 64 * (NCH * wave + n) + lane;  // physical 16-byte chunk of the tile
      const int krow = P >> 3, kc = (P & 7) ^ ((krow >> 1) & 7);
      kdma[n] = (uint32_t)(krow * FD + kc * 16);
      const int vrow = P >> 2, vc = (P & 3) ^ ((vrow >> 2) & 3);
      vdma[n] = (uint32_t)vrow * (uint32_t)Sp + (uint32_t)(vc * 16);
    }
  }
};

template <bool MASK>
__device__ __forceinline__ float fp8_tile_max(f32x16 (&s)[2], int k0, int lim, int hh) {
  float mx = kNegInf;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if (MASK) {
        const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (key > lim) s[kb][r] = kNegInf;
      }
      mx = __builtin_fmaxf(mx, s[kb][r]);
    }
  }
  return __builtin_fmaxf(mx, wave_swap_halves(mx));
}

// NW wavefronts (4 or 8) of 32 query rows each share every K / V tile.
template <int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void fwd_fp8_kernel(Fp8Buf f, uint16_t* __restrict__ O,
                                                                float* __restrict__ LSE, int BH, int S, int nqt,
                                                                float C, uint32_t qsign, float tau, int causal) {
  constexpr int BR = 32 * NW;         // query rows of the workgroup
  constexpr int NCH = 512 / (64 * NW);  // 16-byte chunks per lane of a tile
  static_assert(NCH * 64 * NW == 512, "a tile is 512 chunks of 16 bytes");
  // one __shared__ array per buffer, chosen at compile time (the loop is
  // unrolled by two): the compiler then sees that a tile load in flight does
  // not alias the buffer being read and does not wait for it
  __shared__ __attribute__((aligned(1024))) uint8_t Kb0[FBC * FD];
  __shared__ __attribute__((aligned(1024))) uint8_t Kb1[FBC * FD];
  __shared__ __attribute__((aligned(1024))) uint8_t Vb0[FD * FBC];
  __shared__ __attribute__((aligned(1024))) uint8_t Vb1[FD * FBC];

  const int Sp = f.Sp;
  // block order (xcd_head_order): one head's query tiles together on an XCD
  // in non-causal passes (same-process A/B: 1.1 % faster at S = 8192, 2.9 %
  // at S = 32768); causal passes run the heaviest query tiles of all heads
  // first (the grouped order measured 1.1 % slower at S = 32768)
  int bh, rank;
  xcd_head_order(blockIdx.x, BH, nqt, !causal, bh, rank);
  const int qt = causal ? (nqt - 1 - rank) : rank;
  const int q0 = qt * BR;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  // the same index read from the first lane, for the LDS-DMA destinations only
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int lane = tid & 63;
  const int hh = lane >> 5;
  const int c32 = lane & 31;
  const int qw0 = q0 + 32 * wave;
  const int qrow = qw0 + c32;
  // rows past the padded length (eight wavefronts, Sp an odd multiple of
  // 128) read the last padded row and store nothing
  const int qread = min(qrow, Sp - 1);
  const uint8_t* Kh = f.k8 + (size_t)bh * Sp * FD;
  const uint8_t* Vh = f.v8t + (size_t)bh * FD * Sp;

  // Q^T operand: lane holds bytes 64 t + 32 hh .. + 31 of row qrow
  i32x8 qreg[2];
  {
    const uint8_t* qp = f.q8 + ((size_t)bh * Sp + qread) * FD;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      u32x4 a = *reinterpret_cast<const u32x4*>(qp + 64 * t + 32 * hh);
      u32x4 b = *reinterpret_cast<const u32x4*>(qp + 64 * t + 32 * hh + 16);
      a ^= qsign;  // a negative scale flips the sign of every Q code
      b ^= qsign;
      qreg[t] = i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
    }
  }
  // scale * log2(e) * this row's Q scale * the head's K scale: the score
  // factor of every tile (log2 units)
  const float ct = C * f.qs[(size_t)bh * Sp + qread] * f.ks[bh];

  const int kend = causal ? min(S, q0 + BR) : S;
  const int nkt = (kend + FBC - 1) / FBC;
  const int wend = causal ? min(kend, qw0 + 32) : kend;
  const int nkt_w = qw0 < S ? (wend + FBC - 1) / FBC : 0;
  int nfull = causal ? (qw0 + 1) / FBC : nkt_w;
  nfull = max(0, min(nfull, S / FBC));
  const int lim = causal ? min(qrow, S - 1) : (S - 1);

  Fp8Wave of;
  of.init<NCH>(wave, lane, Sp);

  // extent: bytes of the head's array from the tile start on
  auto dma = [&](const uint8_t* src, uint32_t extent, uint8_t* dst, const uint32_t (&off)[2]) {
#pragma unroll
    for (int n = 0; n < NCH; ++n) lds_dma<16>(src, extent, off[n], dst + 1024 * (NCH * wave_u + n));
  };
  // iteration j issues K(j + 2) and V(j + 1) into the buffers the barrier of
  // iteration j - 1 freed; it reads K(j + 1) (scores of the next tile) and V(j)
  const uint32_t head_bytes = (uint32_t)Sp * FD;
  auto issue = [&](int j, auto P) {  // P = j & 1
    constexpr int par = decltype(P)::value;
    if (j + 2 < nkt)
      dma(Kh + (size_t)(j + 2) * FBC * FD, head_bytes - (uint32_t)((j + 2) * FBC * FD), par ? Kb1 : Kb0, of.kdma);
    if (j + 1 >= 0 && j + 1 < nkt)
      dma(Vh + (size_t)(j + 1) * FBC, head_bytes - (uint32_t)((j + 1) * FBC), par ? Vb0 : Vb1, of.vdma);
  };
  auto scores = [&](const uint8_t* kb_, f32x16 (&s)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
#pragma unroll
      for (int t = 0; t < 2; ++t)
        s[kb] = mfma_fp8(lds_frag32(kb_ + 32 * kb * FD + of.kfrag[t][0], kb_ + 32 * kb * FD + of.kfrag[t][1]), qreg[t],
                         s[kb]);
    }
  };

  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) oacc[db] = f32x16{};
  float m_run = kNegInf;  // running max in log2 units
  float l_part = 0.0f;    // this lane's partial row sum (unrounded P)

  issue(-2, std::integral_constant<int, 0>{});
  issue(-1, std::integral_constant<int, 1>{});
  wait_vm_lds<0>();
  __syncthreads();
  f32x16 sa[2], sb[2];
  scores(Kb0, sa);
  wait_vm_lds<63>();
  barrier_keep_loads();

  auto step = [&](auto maskc, auto P, int kt, f32x16(&scur)[2], f32x16(&snext)[2]) {
    constexpr int par = decltype(P)::value;  // kt & 1
    constexpr bool MASK = decltype(maskc)::value;
    // distinct code at the top of each copy: keeps the compiler from hoisting
    // the two copies' common reads out of the masked / unmasked branch
    tile_marker<MASK>();
    // Region 1 (raised wave priority): the next tile's four score MFMAs
    // interleaved with this tile's softmax.  Back to back, each MFMA would
    // hold the wavefront until the previous one leaves the matrix pipe.
    __builtin_amdgcn_s_setprio(1);
    scores(par ? Kb0 : Kb1, snext);
    const float mx = fp8_tile_max<MASK>(scur, kt * FBC, lim, hh);
    const float mxs = (mx == kNegInf) ? kNegInf : mx * ct;
    const float m_new = __builtin_fmaxf(m_run, mxs);
    const bool grow = __any((m_new - m_run) > tau);
    // no branch here: exp2(0) = 1 when the max does not move (a branch would
    // split the region and stop the scheduler from interleaving it)
    const float alpha = exp2_native((grow && m_new != kNegInf) ? (m_run - m_new) : 0.0f);
    m_run = grow ? m_new : m_run;
    l_part *= alpha;
    // P = exp2(S ct - m) to E4M3: byte 16 kb + r of the operand is register r
    // of block kb, the key order of V^T in LDS
    i32x8 pf;
    const float negm = -m_run;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int w4 = 0; w4 < 4; ++w4) {
        float p[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * w4 + e;
          float x = exp2_native(__builtin_fmaf(scur[kb][r], ct, negm));
          if (MASK && scur[kb][r] == kNegInf) x = 0.0f;
          p[e] = x;
          l_part += x;
        }
        pf[4 * kb + w4] = (int)pack_e4m3x4(p[0], p[1], p[2], p[3]);
      }
    }
    // the K fragment reads first, the tile max under their latency, then
    // each MFMA followed by a share of the softmax (VALU and exponentials)
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
    __builtin_amdgcn_sched_group_barrier(0x402, 40, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x402, 26, 0);
    }
    // keep P and the row sum above the (rare) rescale branch: otherwise the
    // compiler sinks them next to the PV products, out of this schedule
#pragma unroll
    for (int w = 0; w < 8; ++w) asm volatile("" ::"v"(pf[w]));
    asm volatile("" ::"v"(l_part));
    __builtin_amdgcn_s_setprio(0);
    if (grow) {
#pragma unroll
      for (int db = 0; db < 4; ++db) oacc[db] *= alpha;
    }
    const uint8_t* vb = par ? Vb1 : Vb0;
#pragma unroll
    for (int db = 0; db < 4; ++db)
      oacc[db] = mfma_fp8(lds_frag32(vb + 32 * db * FBC + of.vfrag[0], vb + 32 * db * FBC + of.vfrag[1]), pf, oacc[db]);
  };

  auto iteration = [&](int kt, auto P, f32x16(&scur)[2], f32x16(&snext)[2]) {
    issue(kt, P);
    __builtin_amdgcn_sched_barrier(0);
    if (kt < nkt_w) {
      if (kt < nfull)
        step(std::false_type{}, P, kt, scur, snext);
      else
        step(std::true_type{}, P, kt, scur, snext);
    }
    wait_vm_lds<0>();
    barrier_keep_loads();
  };
  for (int kt = 0; kt < nkt; kt += 2) {
    iteration(kt, std::integral_constant<int, 0>{}, sa, sb);
    if (kt + 1 < nkt) iteration(kt + 1, std::integral_constant<int, 1>{}, sb, sa);
  }

  // ---- epilogue: O = acc * vs / l, LSE = ln2 * (m + log2 l) ----------------
  const float l_tot = l_part + wave_swap_halves(l_part);
  const float inv = 1.0f / l_tot;
  if (qrow < S) {
    const float* vsh = f.vs + (size_t)bh * FD;
    uint16_t* orow = O + ((size_t)bh * S + qrow) * FD;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * db + 8 * g + 4 * hh;
        const f32x4 s4 = *reinterpret_cast<const f32x4*>(vsh + d) * inv;
        *reinterpret_cast<u32x2*>(orow + d) = pack_bf16x4(oacc[db][4 * g] * s4[0], oacc[db][4 * g + 1] * s4[1],
                                                          oacc[db][4 * g + 2] * s4[2], oacc[db][4 * g + 3] * s4[3]);
      }
    }
    if (hh == 0) LSE[(size_t)bh * S + qrow] = (m_run + __log2f(l_tot)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// Diagnostic: the forward kernel's score product on given codes.  Wavefront
// w computes C_w = A_w B_w for an A_w of 32 x 128 codes (row-major) and a
// B_w of 128 x 32 codes given transposed (Bt_w, 32 x 128, row-major), as
// two chained v_mfma_f32_32x32x64_f8f6f4 with the operand layout of
// fwd_fp8_kernel's S^T = K Q^T (lane half h and byte j of both operands
// carry contraction index 64 t + 32 h + j).  C_w is 32 x 32 fp32, row-major.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void fp8_dot_eval_kernel(const uint8_t* __restrict__ A,
                                                           const uint8_t* __restrict__ Bt, float* __restrict__ C,
                                                           long nblk) {
  const long w = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= nblk) return;  // whole wavefronts
  const int lane = threadIdx.x & 63, hh = lane >> 5, c32 = lane & 31;
  const uint8_t* a = A + (size_t)w * 32 * FD + (size_t)c32 * FD;
  const uint8_t* b = Bt + (size_t)w * 32 * FD + (size_t)c32 * FD;
  f32x16 acc = f32x16{};
#pragma unroll
  for (int t = 0; t < 2; ++t)
    acc = mfma_fp8(lds_frag32(a + 64 * t + 32 * hh, a + 64 * t + 32 * hh + 16),
                   lds_frag32(b + 64 * t + 32 * hh, b + 64 * t + 32 * hh + 16), acc);
  float* c = C + (size_t)w * 32 * 32;
#pragma unroll
  for (int r = 0; r < 16; ++r) c[(8 * (r >> 2) + 4 * hh + (r & 3)) * 32 + c32] = acc[r];
}

}  // namespace

size_t fp8_layout(int B, int H, int S, int D, void* base, Fp8Buf* f) {
  (void)D;
  auto r256 = [](size_t n) { return (n + 255) & ~(size_t)255; };
  const size_t BH = (size_t)B * H;
  const int Sp = (S + FBR - 1) / FBR * FBR;
  const size_t vmax_bytes = r256(BH * FD * sizeof(float));
  const size_t sz[7] = {r256(BH * Sp * FD),             // q8
                        r256(BH * Sp * FD),             // k8
                        r256(BH * FD * Sp),             // v8t
                        r256(BH * Sp * sizeof(float)),  // qs
                        r256(BH * sizeof(float)),       // ks
                        r256(BH * FD * sizeof(float)),  // vs
                        vmax_bytes + r256(BH * sizeof(double))};  // scratch: V column maxima, K head maxima
  size_t off[7], total = 0;
  for (int i = 0; i < 7; ++i) {
    off[i] = total;
    total += sz[i];
  }
  if (f != nullptr) {
    char* p = static_cast<char*>(base);
    f->Sp = Sp;
    f->q8 = reinterpret_cast<uint8_t*>(p + off[0]);
    f->k8 = reinterpret_cast<uint8_t*>(p + off[1]);
    f->v8t = reinterpret_cast<uint8_t*>(p + off[2]);
    f->qs = reinterpret_cast<float*>(p + off[3]);
    f->ks = reinterpret_cast<float*>(p + off[4]);
    f->vs = reinterpret_cast<float*>(p + off[5]);
    f->vpart = reinterpret_cast<float*>(p + off[6]);
    f->kmax = reinterpret_cast<void*>(p + off[6] + vmax_bytes);
    for (int i = 0; i < 7; ++i) f->offsets[i] = off[i];
  }
  return total;
}

hipError_t launch_fp8_quantize(const void* Q, const void* K, const void* V, const float* signs, const Fp8Buf& f,
                               int B, int H, int S, hipStream_t st) {
  const int BH = B * H;
  prof_begin(KID_FP8_QUANT, st);
  hipLaunchKernelGGL(fp8_clear_kernel, dim3((BH * FD + 255) / 256), dim3(256), 0, st, f, BH);
  hipLaunchKernelGGL(fp8_qk_quant_kernel<0>, dim3(f.Sp / 64, BH, 1), dim3(256), 0, st, (const uint16_t*)Q,
                     (const uint16_t*)K, signs, f, S);
  hipLaunchKernelGGL(fp8_v_amax_kernel, dim3(f.Sp / 128, BH), dim3(256), 0, st, (const uint16_t*)V, f, S);
  hipLaunchKernelGGL(fp8_qk_quant_kernel<1>, dim3(f.Sp / 64, BH, 2), dim3(256), 0, st, (const uint16_t*)Q,
                     (const uint16_t*)K, signs, f, S);
  hipLaunchKernelGGL(fp8_v_quant_kernel, dim3(f.Sp / 64, BH), dim3(256), 0, st, (const uint16_t*)V, f, S);
  prof_end(KID_FP8_QUANT, st);
  return hipGetLastError();
}

hipError_t launch_fp8_dot_eval(const void* A, const void* Bt, float* C, long nblk, hipStream_t st) {
  hipLaunchKernelGGL(fp8_dot_eval_kernel, dim3((unsigned)((nblk + 3) / 4)), dim3(256), 0, st, (const uint8_t*)A,
                     (const uint8_t*)Bt, C, nblk);
  return hipGetLastError();
}

hipError_t launch_fwd_fp8(const Fp8Buf& f, void* O, float* LSE, int B, int H, int S, float C, uint32_t qsign,
                          float tau, int causal, hipStream_t st) {
  const int BH = B * H;
  const int nqt = (f.Sp + 127) / 128;  // four wavefronts, 128 query rows per workgroup
  prof_begin(KID_FWD_FP8, st);
  hipLaunchKernelGGL(fwd_fp8_kernel<4>, dim3(nqt * BH), dim3(256), 0, st, f, (uint16_t*)O, LSE, BH, S, nqt, C,
                     qsign, tau, causal);
  prof_end(KID_FWD_FP8, st);
  return hipGetLastError();
}

}  // namespace attn97

// attn_bwd.hip - backward pass of exact attention on gfx950: the dK/dV
// kernels (split mode; with dQ by fp32 atomics in the atomic mode) and the
// launch logic of both modes.
//
// The forward pass stored only O and the row log-sum-exp, so the backward
// pass recomputes the probabilities from them:
//
//   Delta_i = sum_d dO_id O_id                       (bwd_pre_kernel; in the
//                                                       split mode the dQ kernel)
//   P  = exp2(S * scale*log2e - LSE*log2e),  S = Q K^T   (-LSE log2e likewise)
//   dV += P^T dO,   dP = dO V^T,   dS = P * (dP - Delta)
//   dK += dS^T Q,   dQ += dS K                       (bwd_main_kernel)
//   dQ (bf16) = fp32 accumulator                     (dq_convert_kernel)
//
// scale is applied to dK at the end and to each dQ contribution.  The pages
// give no backward equations; these follow from the chain rule on
// O = softmax(scale Q K^T) V.  The pages do say where the backward pass
// spends its time: shared-memory traffic and the atomic additions that
// accumulate dQ (page "FlashAttention-4 : comment Together AI a accéléré
// l'attention sur GPU Blackwell", sections "Pourquoi l'approche standard ne
// fonctionne plus" and "Les capacités de Blackwell qui l'ont rendu possible";
// page "FlashAttention-3 и FlashAttention-4", section "Режим 2-CTA MMA").
//
// bwd_main_kernel: one workgroup of four wavefronts owns 128 keys of one
// (batch, head); each wavefront owns 32 keys, keeps their K and V rows in
// registers as MFMA operands and their dK, dV accumulators in registers, and
// walks the query sequence one tile of BQ rows at a time.  Scores are
// computed as S[q, key] so that each lane holds one key column: P and dS
// then feed the dV and dK products straight from registers (as P^T, dS^T).
// The dQ product needs dS with queries as rows, so dS goes through LDS once
// (bf16); each wavefront then forms a 32x32 block of the tile's dQ over all
// 128 keys and adds it to an fp32 accumulator in global memory.
#include <stdlib.h>

#include <type_traits>

#include "attn_kernels.hpp"
#include "device_common.hpp"
#include "tile_layout.hpp"

namespace attn97 {

template <int D, int BQ_ = 64>
struct BwdCfg {
  static constexpr int NW = 4;                     // wavefronts per workgroup
  static constexpr int BK = 32 * NW;               // keys per workgroup
  static constexpr int BQ = BQ_;                   // queries per tile
  static constexpr int NQB = BQ / 32;              // 32-query blocks per tile
  static constexpr int NKS = D / 16;               // reduction steps over D
  static constexpr int NDB = D / 32;               // 32-wide blocks of D
  static constexpr int CPR = D / 8;                // 16-byte chunks per row
  static constexpr int SRS = BK + 8;               // row stride of dSs (elements)
  static constexpr int NDQ = NQB * NDB / NW;       // dQ blocks per wavefront
  static constexpr int QTILE = BQ * D;             // elements of a Q or dO tile
  static constexpr int KTILE = BK * D;             // elements of the K tile
  static constexpr int DMA_Q = QTILE * 2 / 1024 / NW;  // 1 KiB loads per wave per Q (or dO) tile
  static constexpr int DMA_K = KTILE * 2 / 1024 / NW;  // ... for the K (or V) tile
  static constexpr int LROWS = BQ < 64 ? 64 : BQ;      // LSE / Delta staging (64 lanes load 64 floats)
  static_assert(DMA_Q >= 1 && DMA_Q * 1024 * NW == QTILE * 2, "Q tile split over waves");
};

// LDS of the backward main kernel.  With dQ (atomic mode) it also holds the
// workgroup's K tile and the bf16 dS tile of the dQ product.
template <class Cfg, bool WITH_DQ, bool VLDS>
struct BwdSmem {
  uint16_t Qs[2][Cfg::QTILE];   // swizzled row-major Q tiles (double buffer)
  uint16_t dOs[2][Cfg::QTILE];  // swizzled row-major dO tiles
  uint16_t Ks[Cfg::KTILE];      // swizzled row-major K tile of the workgroup
  uint16_t dSs[Cfg::BQ * Cfg::SRS];
  float lse[2][Cfg::LROWS];  // -LSE log2(e) of the tile's rows
  float dlt[2][Cfg::LROWS];
};
// Without dQ (split mode): Q / dO tiles, LSE / Delta and, with VLDS, the
// workgroup's V tile (otherwise V rows are held in registers).
template <class Cfg>
struct BwdSmem<Cfg, false, true> {
  uint16_t Qs[2][Cfg::QTILE];
  uint16_t dOs[2][Cfg::QTILE];
  uint16_t Vs[Cfg::KTILE];  // swizzled row-major V tile of the workgroup
  float lse[2][Cfg::LROWS];
  float dlt[2][Cfg::LROWS];
};
template <class Cfg>
struct BwdSmem<Cfg, false, false> {
  uint16_t Qs[2][Cfg::QTILE];
  uint16_t dOs[2][Cfg::QTILE];
  float lse[2][Cfg::LROWS];
  float dlt[2][Cfg::LROWS];
};

// Exchange with the neighbouring lane (l ^ 1) through DPP (quad_perm 1,0,3,2).
__device__ __forceinline__ float swap_lane_pair(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

// Epilogue of the dK / dV kernels.  The accumulators hold one column per
// lane (16 keys per lane and 32-column block); stored straight out that is
// one 2-byte store per lane and element.  Instead the wavefront stages its 32
// keys x DW columns as bf16 in its own LDS slice (row-major, stride DW) and
// stores whole 16-byte chunks of rows: DW / 16 stores per matrix instead of
// 16 NDO.  dK is multiplied by `scale`.  The slice is reused for dV once
// dK's rows have been read back (the LDS operations of one wavefront
// complete in issue order).  dKw / dVw: row 0 of the wavefront's keys at its
// first column; ld: row stride (elements); rows at or past nrows are not
// stored.
template <int NDO>
__device__ __forceinline__ void store_dkdv_rows(const f32x16 (&dk)[NDO], const f32x16 (&dv)[NDO], float scale,
                                                uint16_t* slice, uint16_t* dKw, uint16_t* dVw, int ld, int nrows,
                                                int lane) {
  constexpr int DW = 32 * NDO, CPR = DW / 8, RPI = 64 / CPR;
  static_assert(64 % CPR == 0 && 32 % RPI == 0, "whole rows per store");
  const int hh = lane >> 5, c32 = lane & 31;
  const int rr = lane / CPR, c8 = (lane % CPR) * 8;
#pragma unroll
  for (int m = 0; m < 2; ++m) {
#pragma unroll
    for (int db = 0; db < NDO; ++db) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float x = m == 0 ? dk[db][r] * scale : dv[db][r];
        slice[(8 * (r >> 2) + 4 * hh + (r & 3)) * DW + 32 * db + c32] = __builtin_bit_cast(uint16_t, (__bf16)x);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    uint16_t* dst = m == 0 ? dKw : dVw;
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int row = i * RPI + rr;
      const u32x4 v = *reinterpret_cast<const u32x4*>(slice + row * DW + c8);
      if (row < nrows) *reinterpret_cast<u32x4*>(dst + (size_t)row * ld + c8) = v;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// Two LDS transpose loads (four rows each, at this lane's column) as one
// MFMA operand.
__device__ __forceinline__ bf16x8 tr_operand(const uint16_t* p0, const uint16_t* p1) {
  const s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p0));
  const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p1));
  const s16x8 v = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// p advanced by `bytes` (the per-lane offsets below are byte offsets, so an
// LDS address is the offset plus the tile's base as the instruction's
// immediate, with no shift per use).
__device__ __forceinline__ const uint16_t* at_bytes(const uint16_t* p, uint32_t bytes) {
  return reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(p) + bytes);
}

// Per-lane LDS and DMA offsets (bytes) fixed over the whole kernel.
template <int D, class Cfg>
struct BwdOffsets {
  static constexpr int NKS = Cfg::NKS, NDB = Cfg::NDB;
  // A operand of S = Q K^T and dP = dO V^T: row c32 (+32 qb), chunk 2 ks + h.
  int arow[NKS];
  // B operand of dV += P^T dO and dK += dS^T Q (q contraction, rows permuted
  // like the P / dS registers): rows 8 r2 + 4 h + (i >> 2) (+16 t).
  int trq[NDB][2];
  // B operand of dQ += dS K (key contraction, natural key order): rows
  // 8 h + 4 r2 + (i >> 2) (+16 t).
  int trk[NDB][2];
  uint32_t dmaq[Cfg::DMA_Q];
  uint32_t dmak[Cfg::DMA_K];

  // d0: first column of the dK / dV block this workgroup forms (the
  // transpose-read offsets start there; 0 unless the columns are split).
  __device__ __forceinline__ void init(int wave, int lane, int d0 = 0) {
    const int hh = lane >> 5, c32 = lane & 31, i = lane & 15, g16 = lane >> 4;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) arow[ks] = swz_chunk<D>(c32, 2 * ks + hh) * 16;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int d = d0 + 32 * db + 16 * (g16 & 1) + 4 * (i & 3);
#pragma unroll
      for (int r2 = 0; r2 < 2; ++r2) {
        trq[db][r2] = (swz_chunk<D>(8 * r2 + 4 * (g16 >> 1) + (i >> 2), d >> 3) * 8 + (d & 7)) * 2;
        trk[db][r2] = (swz_chunk<D>(8 * (g16 >> 1) + 4 * r2 + (i >> 2), d >> 3) * 8 + (d & 7)) * 2;
      }
    }
#pragma unroll
    for (int n = 0; n < Cfg::DMA_Q; ++n) {
      int row, c;
      unswz_chunk<D>(64 * (wave * Cfg::DMA_Q + n) + lane, row, c);
      dmaq[n] = (uint32_t)(row * D + 8 * c) * 2;
    }
#pragma unroll
    for (int n = 0; n < Cfg::DMA_K; ++n) {
      int row, c;
      unswz_chunk<D>(64 * (wave * Cfg::DMA_K + n) + lane, row, c);
      dmak[n] = (uint32_t)(row * D + 8 * c) * 2;
    }
  }
};

// Load rows r0.. of a [S, D] bf16 matrix into a swizzled LDS tile with
// buffer loads with the LDS bit (lds_dma); rows past S are clamped to S-1
// (finite data, masked later).  `loff` are this lane's logical byte offsets
// inside the tile; dma_row_part issues this wave's n-th 1 KiB piece only.
// CLAMP = false: the caller guarantees r0 + rows <= S (no clamp code).
template <int D, int NPW, bool CLAMP = true>
__device__ __forceinline__ void dma_row_part(const uint16_t* __restrict__ src, int r0, int rows, int S, uint16_t* dst,
                                             int wave, const uint32_t (&loff)[NPW], int n) {
  const uint16_t* tile = src + (size_t)r0 * D;
  uint32_t off = loff[n];  // bytes
  if (CLAMP && r0 + rows > S) {
    const uint32_t row = off / (2 * D);
    const uint32_t last = (uint32_t)(S - 1 - r0);
    off = (row > last ? last : row) * (2 * D) + off % (2 * D);
  }
  lds_dma<16>(tile, (uint32_t)(S > r0 ? S - r0 : 0) * (uint32_t)(D * 2), off, dst + 512 * (wave * NPW + n));
}

// The same piece at a given byte offset `off` (rows past S load as zeros).
template <int D, int NPW>
__device__ __forceinline__ void dma_row_at(const uint16_t* __restrict__ src, int r0, int S, uint16_t* dst, int wave,
                                           int n, uint32_t off) {
  lds_dma<16>(src + (size_t)r0 * D, (uint32_t)(S > r0 ? S - r0 : 0) * (uint32_t)(D * 2), off,
              dst + 512 * (wave * NPW + n));
}

// Closed form of BwdOffsets::dmaq[n] at D = 128 and 256 (16 rows per wave's
// pieces, 64 / (D / 8) rows per piece): with lr = lane / (D / 8) and
// cc = lane % (D / 8), piece n's offset is y + 1024 n + 16 (x ^ g(n)) for the
// per-lane values x = cc ^ 4 lr and y = 32 D wave + 2 D lr, where g(n) is the
// swizzle term of the piece's rows; the two fields of the swizzle's XOR land
// in disjoint bits, so the lane's part folds into x.
template <int D>
__device__ __forceinline__ uint32_t dmaq_closed(uint32_t x, uint32_t y, int n) {
  static_assert(D == 128 || D == 256, "rows of 256 or 512 bytes");
  const uint32_t g = D == 128 ? (uint32_t)n : (uint32_t)(8 * (n & 1) + (n >> 1));
  return y + 1024u * (uint32_t)n + 16u * (x ^ g);
}

template <int D, int NPW, bool CLAMP = true>
__device__ __forceinline__ void dma_rows(const uint16_t* __restrict__ src, int r0, int rows, int S, uint16_t* dst,
                                         int wave, const uint32_t (&loff)[NPW]) {
#pragma unroll
  for (int n = 0; n < NPW; ++n) dma_row_part<D, NPW, CLAMP>(src, r0, rows, S, dst, wave, loff, n);
}

// One query tile against one wavefront's 32 keys: S = Q K^T and dP = dO V^T,
// P = exp2(S c - LSE log2e), dS = P (dP - Delta), dS to LDS (queries as rows)
// for the dQ product, then dV += P^T dO and dK += dS^T Q with the q-major
// operands read by LDS transpose loads.  need_mask (wave-uniform) applies
// the diagonal / ragged mask after the exponentials; one code path serves
// every tile, so the operand reads stay inside the step's read-ahead
// schedule.
// NDO: 32-wide column blocks of dK / dV this wavefront accumulates (D / 32,
// or fewer when the workgroups split the columns; the offsets then start at
// the block's first column).
template <int D, class Cfg, bool CAUSAL, bool WRITE_DS, bool VLDS, int NDO>
__device__ __forceinline__ void bwd_tile(BwdSmem<Cfg, WRITE_DS, VLDS>& sm, int buf, const BwdOffsets<D, Cfg>& of,
                                         const bf16x8 (&kreg)[D / 16], const bf16x8 (&vreg)[VLDS ? 1 : D / 16],
                                         const uint16_t* Vw, f32x16 (&dk)[NDO], f32x16 (&dv)[NDO], int q0,
                                         int key, int S, float C, int c32, int hh, int dsw, bool need_mask) {
  constexpr int NQB = Cfg::NQB, NKS = Cfg::NKS, NDB = NDO, SRS = Cfg::SRS, CPR = Cfg::CPR;
  const uint16_t* Qb = sm.Qs[buf];
  const uint16_t* dOb = sm.dOs[buf];
  const bool odd = c32 & 1;
  // Register (qb, g, e) holds query q0 + 4 hh + c, c = 32 qb + 8 g + e.  It
  // is kept iff that query is < S, this lane's key is < S and (causal)
  // key <= query: as a range of the constant part, mlo <= c < mhi.
  const int mt = q0 + 4 * hh;
  const int mlo = CAUSAL ? key - mt : 0;
  const int mhi = key < S ? S - mt : -1;
  bf16x8 pb[2 * NQB], dsb[2 * NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    f32x16 sacc = f32x16{}, dpacc = f32x16{};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      sacc = mfma32(lds_frag(at_bytes(Qb, of.arow[ks]) + 32 * qb * CPR * 8), kreg[ks], sacc);
      if constexpr (VLDS)
        dpacc = mfma32(lds_frag(at_bytes(dOb, of.arow[ks]) + 32 * qb * CPR * 8), lds_frag(at_bytes(Vw, of.arow[ks])), dpacc);
      else
        dpacc = mfma32(lds_frag(at_bytes(dOb, of.arow[ks]) + 32 * qb * CPR * 8), vreg[ks], dpacc);
    }
    // two reduction steps of operands read ahead of the MFMAs (Q, dO and,
    // with VLDS, V fragments: 2 or 3 LDS reads per step of two MFMAs)
    if constexpr (VLDS) {
      __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
      for (int i = 0; i < NKS - 2; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    } else {
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < 2 * NKS - 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    float p[16], ds[16];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int qr = 32 * qb + 8 * g + 4 * hh;  // tile row of register 4g
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(&sm.lse[buf][qr]);
#pragma unroll
      for (int e = 0; e < 4; ++e) p[4 * g + e] = exp2_native(__builtin_fmaf(sacc[4 * g + e], C, l4[e]));
    }
    if (need_mask) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int c = 32 * qb + 8 * (r >> 2) + (r & 3);
        if (!(c >= mlo && c < mhi)) p[r] = 0.0f;
      }
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(&sm.dlt[buf][32 * qb + 8 * g + 4 * hh]);
#pragma unroll
      for (int e = 0; e < 4; ++e) ds[4 * g + e] = p[4 * g + e] * (dpacc[4 * g + e] - d4[e]);
    }
    pb[2 * qb] = to_bf16x8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
    pb[2 * qb + 1] = to_bf16x8(p[8], p[9], p[10], p[11], p[12], p[13], p[14], p[15]);
    dsb[2 * qb] = to_bf16x8(ds[0], ds[1], ds[2], ds[3], ds[4], ds[5], ds[6], ds[7]);
    dsb[2 * qb + 1] = to_bf16x8(ds[8], ds[9], ds[10], ds[11], ds[12], ds[13], ds[14], ds[15]);
    // dS to LDS with queries as rows and keys in natural order.  Lanes l and
    // l^1 hold adjacent keys; for rows (r, r+1) the even lane writes row r
    // and the odd lane row r+1, each as one 32-bit pair of adjacent keys
    // (dsw holds the odd lane's one-row offset and the even key column).
    if constexpr (WRITE_DS) {
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float recv = swap_lane_pair(odd ? ds[r] : ds[r + 1]);
        const float lo = odd ? recv : ds[r];
        const float hi = odd ? ds[r + 1] : recv;
        const int row = 32 * qb + 8 * (r >> 2) + 4 * hh + (r & 3);
        *reinterpret_cast<uint32_t*>(&sm.dSs[row * SRS + dsw]) = pack_bf16x2(lo, hi);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < 2 * NQB; ++t) {
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int o = 16 * t * CPR * 8;
      dv[db] = mfma32(pb[t], tr_operand(at_bytes(dOb, of.trq[db][0]) + o, at_bytes(dOb, of.trq[db][1]) + o), dv[db]);
      dk[db] = mfma32(dsb[t], tr_operand(at_bytes(Qb, of.trq[db][0]) + o, at_bytes(Qb, of.trq[db][1]) + o), dk[db]);
    }
  }
  __builtin_amdgcn_sched_group_barrier(0x100, 8, 1);
#pragma unroll
  for (int i = 0; i < 4 * NQB * NDB - 2; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
}

// ---- split mode: one 64-query tile in four software-pipelined phases -------
//
// With one wavefront per SIMD, the matrix unit idles whenever the wavefront
// is busy with the softmax VALU work or waits for an MFMA result.  The tile's
// two 32-query blocks are therefore staggered so that each phase pairs MFMAs
// with independent VALU work of the other block:
//
//   A: S, dP of block 0
//   B: S, dP of block 1        | softmax of block 0 (P, dS -> bf16)
//   C: dV, dK with block 0     | softmax of block 1
//   D: dV, dK with block 1
//
// (the softmax overlapping the matrix products of another block, page
// "FlashAttention-3 и FlashAttention-4", section "Чередование matmul и
// softmax").  Scheduling barriers keep each phase's instructions together and
// interleave them in fixed proportions.

// Qb, dOb, nl, dl: this tile's Q and dO tiles and -LSE log2e / Delta rows in
// LDS.  issue_part(p) issues piece p of the next tile's loads; the pieces go
// out over phases A and B, one every other step (issued back to back they
// fill the memory pipeline and stall the wavefront for hundreds of cycles).
// Hooks of the fused atomic mode (DqHooks in bwd_dkdv_kernel): store(qb,
// dsb) puts block qb's dS (bf16) into LDS once it is formed; step(i), in
// each of phase D's eight steps, runs one k-step of the previous tile's dQ
// product.  NoDq is the split mode's: nothing.
struct NoDq {
  __device__ __forceinline__ void store(int, const bf16x8 (&)[2]) {}
  __device__ __forceinline__ void step(int) {}
};

// D = 128, or D = 256 with the dK / dV columns split between two workgroups
// (NDO: the 32-column output blocks this workgroup forms, four either way).
// At D = 256 the S and dP products take sixteen reduction steps, and phase B
// carries one softmax element per step instead of two.
template <int D, class Cfg, bool CAUSAL, bool MASK, int NDO, class IssuePart, class Dq = NoDq>
__device__ __forceinline__ void dkdv_tile(const uint16_t* Qb, const uint16_t* dOb, const float* nl, const float* dl,
                                          const BwdOffsets<D, Cfg>& of, const bf16x8 (&kreg)[D / 16],
                                          const bf16x8 (&vreg)[D / 16], f32x16 (&dk)[NDO], f32x16 (&dv)[NDO],
                                          int q0, int key, int S, float C, int hh, IssuePart&& issue_part,
                                          Dq&& dq = Dq{}) {
  static_assert(Cfg::NQB == 2 && ((D == 64 && NDO == 2) || ((D == 128 || D == 256) && NDO == 4)),
                "two 32-query blocks; four output blocks (two at D = 64)");
  constexpr int NKS = Cfg::NKS, NDB = NDO, CPR = Cfg::CPR;
  tile_marker<MASK>();
  int mlo = 0, mhi = 0;
  if constexpr (MASK) {  // register (qb, g, e) holds query q0 + 4 hh + 32 qb + 8 g + e
    const int mt = q0 + 4 * hh;
    mlo = CAUSAL ? key - mt : 0;
    mhi = key < S ? S - mt : -1;
  }
  auto qfrag = [&](int qb, int ks) { return lds_frag(at_bytes(Qb, of.arow[ks]) + 32 * qb * CPR * 8); };
  auto dofrag = [&](int qb, int ks) { return lds_frag(at_bytes(dOb, of.arow[ks]) + 32 * qb * CPR * 8); };
  auto trdo = [&](int t, int db) {
    const int o = 16 * t * CPR * 8;
    return tr_operand(at_bytes(dOb, of.trq[db][0]) + o, at_bytes(dOb, of.trq[db][1]) + o);
  };
  auto trq = [&](int t, int db) {
    const int o = 16 * t * CPR * 8;
    return tr_operand(at_bytes(Qb, of.trq[db][0]) + o, at_bytes(Qb, of.trq[db][1]) + o);
  };

  // the dP accumulators start from Delta (rows 8 g + 4 hh + e of each block)
  auto delta_init = [&](int qb) {
    f32x16 acc;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(&dl[32 * qb + 8 * g + 4 * hh]);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[4 * g + e] = d4[e];
    }
    return acc;
  };
  f32x16 s0 = f32x16{}, dp0 = delta_init(0), s1 = f32x16{}, dp1;
  uint32_t pw[8], gw[8];  // P / dS of a block, two bf16 per register as they are formed
  float pe = 0.f, ge = 0.f;
  auto put = [&](int r, float pv, float gv) {
    if (r & 1) {
      pw[r >> 1] = pack_bf16x2(pe, pv);
      gw[r >> 1] = pack_bf16x2(ge, gv);
    } else {
      pe = pv;
      ge = gv;
    }
  };
  auto packed = [&](bf16x8 (&pb)[2], bf16x8 (&gb)[2]) {
    pb[0] = __builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]});
    pb[1] = __builtin_bit_cast(bf16x8, u32x4{pw[4], pw[5], pw[6], pw[7]});
    gb[0] = __builtin_bit_cast(bf16x8, u32x4{gw[0], gw[1], gw[2], gw[3]});
    gb[1] = __builtin_bit_cast(bf16x8, u32x4{gw[4], gw[5], gw[6], gw[7]});
  };
  bf16x8 pb0[2], dsb0[2], pb1[2], dsb1[2];

  // A: S, dP of block 0; operand reads two steps ahead
  {
    bf16x8 qa[NKS], da[NKS];
    qa[0] = qfrag(0, 0); da[0] = dofrag(0, 0);
    qa[1] = qfrag(0, 1); da[1] = dofrag(0, 1);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      if (ks + 2 < NKS) { qa[ks + 2] = qfrag(0, ks + 2); da[ks + 2] = dofrag(0, ks + 2); }
      if ((ks & 1) == 0) issue_part(ks / 2);
      if (ks == NKS - 1) dp1 = delta_init(1);
      s0 = mfma32(qa[ks], kreg[ks], s0);
      dp0 = mfma32(da[ks], vreg[ks], dp0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // The softmax of a block runs as a three-stage software pipeline over the
  // eight steps of a phase, two elements per step: step k forms the exponent
  // argument of step k + 1's elements, exponentiates step k's and forms dS of
  // step k - 1's, so that no instruction waits on the one just before it and
  // the MFMAs issue on time.  tt: arguments, pp: P.
  float tt[16], pp[16];
  auto sm_arg = [&](const f32x16& sacc, const f32x4 (&l4)[4], int r) {
    tt[r] = __builtin_fmaf(sacc[r], C, l4[(r >> 2) & 3][r & 3]);
  };
  auto sm_exp = [&](int r, int c) {
    float pv = exp2_native(tt[r]);
    if (MASK) pv = (c >= mlo && c < mhi) ? pv : 0.0f;
    pp[r] = pv;
  };
  auto sm_ds = [&](const f32x16& ndacc, int r) { put(r, pp[r], -pp[r] * ndacc[r]); };

  // B: S, dP of block 1, each step with two elements of block 0's softmax
  // (D = 256: one element per step, D = 64: four, the same three stages)
  if constexpr (NKS == 4) {
    bf16x8 qa[NKS], da[NKS];
    f32x4 l4[4];
    qa[0] = qfrag(1, 0); da[0] = dofrag(1, 0);
#pragma unroll
    for (int g = 0; g < 4; ++g) l4[g] = *reinterpret_cast<const f32x4*>(&nl[8 * g + 4 * hh]);
    qa[1] = qfrag(1, 1); da[1] = dofrag(1, 1);
#pragma unroll
    for (int e = 0; e < 4; ++e) sm_arg(s0, l4, e);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {  // elements 4 ks .. 4 ks + 3 (query rows 8 ks + e)
      if (ks + 2 < NKS) { qa[ks + 2] = qfrag(1, ks + 2); da[ks + 2] = dofrag(1, ks + 2); }
      if ((ks & 1) == 0) issue_part(NKS / 2 + ks / 2);
      if (ks == NKS - 1) issue_part(NKS);
      s1 = mfma32(qa[ks], kreg[ks], s1);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (ks + 1 < NKS) sm_arg(s0, l4, 4 * ks + 4 + e);
        sm_exp(4 * ks + e, 8 * ks + e);
      }
      dp1 = mfma32(da[ks], vreg[ks], dp1);
      if (ks >= 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e) sm_ds(dp0, 4 * ks - 4 + e);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) sm_ds(dp0, 12 + e);
    packed(pb0, dsb0);
    dq.store(0, dsb0);
  } else if constexpr (NKS == 16) {
    bf16x8 qa[NKS], da[NKS];
    f32x4 l4[4];
    qa[0] = qfrag(1, 0); da[0] = dofrag(1, 0);
#pragma unroll
    for (int g = 0; g < 4; ++g) l4[g] = *reinterpret_cast<const f32x4*>(&nl[8 * g + 4 * hh]);
    qa[1] = qfrag(1, 1); da[1] = dofrag(1, 1);
    sm_arg(s0, l4, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      if (ks + 2 < NKS) { qa[ks + 2] = qfrag(1, ks + 2); da[ks + 2] = dofrag(1, ks + 2); }
      if ((ks & 1) == 0) issue_part(NKS / 2 + ks / 2);
      if (ks == NKS - 1) issue_part(NKS);
      s1 = mfma32(qa[ks], kreg[ks], s1);
      if (ks + 1 < NKS) sm_arg(s0, l4, ks + 1);
      sm_exp(ks, 8 * (ks >> 2) + (ks & 3));
      dp1 = mfma32(da[ks], vreg[ks], dp1);
      if (ks >= 1) sm_ds(dp0, ks - 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    sm_ds(dp0, 15);
    packed(pb0, dsb0);
    dq.store(0, dsb0);
  } else {
    bf16x8 qa[NKS], da[NKS];
    f32x4 l4[4];
    qa[0] = qfrag(1, 0); da[0] = dofrag(1, 0);
    l4[0] = *reinterpret_cast<const f32x4*>(&nl[4 * hh]);
    l4[1] = *reinterpret_cast<const f32x4*>(&nl[8 + 4 * hh]);
    qa[1] = qfrag(1, 1); da[1] = dofrag(1, 1);
    sm_arg(s0, l4, 0);
    sm_arg(s0, l4, 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      if (ks + 2 < NKS) { qa[ks + 2] = qfrag(1, ks + 2); da[ks + 2] = dofrag(1, ks + 2); }
      if (ks == 1 || ks == 3) {  // rows of elements 8 g .. 8 g + 7 (steps 2 g - 1, 2 g: arguments)
        const int g = ks / 2 + 2;
        l4[g] = *reinterpret_cast<const f32x4*>(&nl[8 * g + 4 * hh]);
      }
      if ((ks & 1) == 0) issue_part(NKS / 2 + ks / 2);
      if (ks == NKS - 1) issue_part(NKS);
      s1 = mfma32(qa[ks], kreg[ks], s1);
      if (ks + 1 < NKS) {
        sm_arg(s0, l4, 2 * ks + 2);
        sm_arg(s0, l4, 2 * ks + 3);
      }
      sm_exp(2 * ks, 8 * (ks >> 1) + 2 * (ks & 1));
      sm_exp(2 * ks + 1, 8 * (ks >> 1) + 2 * (ks & 1) + 1);
      dp1 = mfma32(da[ks], vreg[ks], dp1);
      if (ks >= 1) {
        sm_ds(dp0, 2 * ks - 2);
        sm_ds(dp0, 2 * ks - 1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    sm_ds(dp0, 14);
    sm_ds(dp0, 15);
    packed(pb0, dsb0);
    dq.store(0, dsb0);
  }
  // C: dV, dK with block 0, each MFMA with one element of block 1's softmax
  // (D = 64: two elements per MFMA)
  if constexpr (NDB == 2) {
    bf16x8 ta[2 * NDB], tb[2 * NDB];
    f32x4 l4[4];
    ta[0] = trdo(0, 0); tb[0] = trq(0, 0);
#pragma unroll
    for (int g = 0; g < 4; ++g) l4[g] = *reinterpret_cast<const f32x4*>(&nl[32 + 8 * g + 4 * hh]);
#pragma unroll
    for (int e = 0; e < 4; ++e) sm_arg(s1, l4, e);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 2 * NDB; ++i) {  // i = 2 t + db; elements 4 i .. 4 i + 3
      const int t = i / NDB, db = i % NDB;
      if (i + 1 < 2 * NDB) { ta[i + 1] = trdo((i + 1) / NDB, (i + 1) % NDB); tb[i + 1] = trq((i + 1) / NDB, (i + 1) % NDB); }
      dv[db] = mfma32(pb0[t], ta[i], dv[db]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (i + 1 < 2 * NDB) sm_arg(s1, l4, 4 * i + 4 + e);
        sm_exp(4 * i + e, 32 + 8 * i + e);
      }
      dk[db] = mfma32(dsb0[t], tb[i], dk[db]);
      if (i >= 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e) sm_ds(dp1, 4 * i - 4 + e);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) sm_ds(dp1, 12 + e);
    packed(pb1, dsb1);
    dq.store(1, dsb1);
  } else {
    bf16x8 ta[2 * NDB], tb[2 * NDB];  // [t][db] transposed dO / Q operands
    f32x4 l4[4];
    ta[0] = trdo(0, 0); tb[0] = trq(0, 0);
    l4[0] = *reinterpret_cast<const f32x4*>(&nl[32 + 4 * hh]);
    l4[1] = *reinterpret_cast<const f32x4*>(&nl[32 + 8 + 4 * hh]);
    sm_arg(s1, l4, 0);
    sm_arg(s1, l4, 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 2 * NDB; ++i) {  // i = 4 t + db
      const int t = i / NDB, db = i % NDB;
      if (i + 1 < 2 * NDB) { ta[i + 1] = trdo((i + 1) / NDB, (i + 1) % NDB); tb[i + 1] = trq((i + 1) / NDB, (i + 1) % NDB); }
      if (i == 1 || i == 3) {
        const int g = i / 2 + 2;
        l4[g] = *reinterpret_cast<const f32x4*>(&nl[32 + 8 * g + 4 * hh]);
      }
      dv[db] = mfma32(pb0[t], ta[i], dv[db]);
      if (i + 1 < 2 * NDB) {
        sm_arg(s1, l4, 2 * i + 2);
        sm_arg(s1, l4, 2 * i + 3);
      }
      sm_exp(2 * i, 32 + 8 * (i >> 1) + 2 * (i & 1));
      sm_exp(2 * i + 1, 32 + 8 * (i >> 1) + 2 * (i & 1) + 1);
      dk[db] = mfma32(dsb0[t], tb[i], dk[db]);
      if (i >= 1) {
        sm_ds(dp1, 2 * i - 2);
        sm_ds(dp1, 2 * i - 1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    sm_ds(dp1, 14);
    sm_ds(dp1, 15);
    packed(pb1, dsb1);
    dq.store(1, dsb1);
  }
  // D: dV, dK with block 1 (and, fused, a k-step of the previous tile's dQ
  // per step); transposed operands one step ahead
  {
    bf16x8 ta[2 * NDB], tb[2 * NDB];
    ta[0] = trdo(2, 0); tb[0] = trq(2, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 2 * NDB; ++i) {
      const int t = i / NDB, db = i % NDB;
      if (i + 1 < 2 * NDB) { ta[i + 1] = trdo(2 + (i + 1) / NDB, (i + 1) % NDB); tb[i + 1] = trq(2 + (i + 1) / NDB, (i + 1) % NDB); }
      dv[db] = mfma32(pb1[t], ta[i], dv[db]);
      dk[db] = mfma32(dsb1[t], tb[i], dk[db]);
      dq.step(i);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// WITH_DQ: dQ is summed here with fp32 atomics (one kernel for the whole
// backward pass); without it the kernel forms dK and dV only and a separate
// kernel (attn_bwd_dq.hip) forms dQ.  VLDS (split mode only) reads the V
// operand from an LDS tile instead of registers; OCC is the target number of
// workgroups per compute unit.
// DSPLIT (split mode only): the dK / dV columns are divided among DSPLIT
// workgroups per key tile; each recomputes P and dS over the full head dim
// and accumulates D / DSPLIT columns (D = 256: the full-width accumulators
// do not fit the register file next to the K / V operands).
// RAGGED = false (split mode, S a multiple of BQ): no query tile is partial,
// so the tile loads carry no clamp arithmetic.
template <int D, int BQ_, bool CAUSAL, bool WITH_DQ, bool VLDS, int OCC, int DSPLIT = 1, bool RAGGED = true>
__global__ __launch_bounds__(256, OCC) void bwd_main_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ nlse2, const float* __restrict__ delta,
    float* __restrict__ dq32, uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int BH, int S,
    float scale, float C) {
  using Cfg = BwdCfg<D, BQ_>;
  static_assert(!(WITH_DQ && VLDS), "the atomic kernel keeps V in registers");
  constexpr int BK = Cfg::BK, BQ = Cfg::BQ, NKS = Cfg::NKS, NDB = Cfg::NDB, SRS = Cfg::SRS, NDQ = Cfg::NDQ,
                CPR = Cfg::CPR, DMA_Q = Cfg::DMA_Q, DMA_K = Cfg::DMA_K;
  static_assert(!WITH_DQ || (NDQ >= 1 && Cfg::NQB * NDB == NDQ * Cfg::NW), "dQ blocks split evenly");
  static_assert(DSPLIT == 1 || (!WITH_DQ && NDB % DSPLIT == 0), "column split: split mode, whole blocks");
  constexpr int NDO = NDB / DSPLIT;  // 32-wide dK / dV column blocks of this workgroup

  __shared__ __attribute__((aligned(1024))) BwdSmem<Cfg, WITH_DQ, VLDS> sm;

  // with B*H a multiple of 8 all workgroups of one head (both column parts)
  // land on one XCD
  const int id = blockIdx.x;
  const int bh = id % BH;
  const int part = (id / BH) % DSPLIT;
  const int ktile = id / BH / DSPLIT;  // causal: lowest keys (most work) first
  const int k0 = ktile * BK;
  const int d0 = part * (D / DSPLIT);  // first dK / dV column of this workgroup
  const size_t base = (size_t)bh * (size_t)S * D;
  const uint16_t* Qh = Q + base;
  const uint16_t* Kh = K + base;
  const uint16_t* Vh = V + base;
  const uint16_t* dOh = dO + base;
  const float* LSEh = nlse2 + (size_t)bh * S;
  const float* dlth = delta + (size_t)bh * S;
  float* dqh = dq32 + base;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int hh = lane >> 5;
  const int c32 = lane & 31;
  const int kw0 = k0 + 32 * wave;  // first key of this wavefront
  const int key = kw0 + c32;       // this lane's key (MFMA column)

  BwdOffsets<D, Cfg> of;
  of.init(wave, lane, d0);

  // per-tile loads: Q and dO tiles by all waves, -LSE log2e / Delta (64
  // floats each, 4 bytes per lane, at least BQ of them used) by waves 0 / 1
  auto issue = [&](int qt, int buf) {
    const int q0 = qt * BQ;
    dma_rows<D, DMA_Q, RAGGED>(Qh, q0, BQ, S, sm.Qs[buf], wave, of.dmaq);
    dma_rows<D, DMA_Q, RAGGED>(dOh, q0, BQ, S, sm.dOs[buf], wave, of.dmaq);
    if (wave < 2) {
      const float* src = wave == 0 ? LSEh : dlth;
      float* dst = (wave == 0) ? sm.lse[buf] : sm.dlt[buf];
      lds_dma<4>(src, (uint32_t)S * 4u, (uint32_t)min(q0 + lane, S - 1) * 4u, dst);
    }
  };

  const int nqt = (S + BQ - 1) / BQ;
  const int qt0 = CAUSAL ? (k0 / BQ) : 0;
  // the workgroup's K tile (for dQ), the first query tile
  if constexpr (WITH_DQ) dma_rows<D, DMA_K>(Kh, k0, BK, S, sm.Ks, wave, of.dmak);
  if constexpr (VLDS) dma_rows<D, DMA_K>(Vh, k0, BK, S, sm.Vs, wave, of.dmak);
  issue(qt0, 0);

  // K^T / V^T operands of S = Q K^T and dP = dO V^T: lane holds row `key`.
  // Rows past the end are clamped (finite data); their P is masked to zero.
  bf16x8 kreg[NKS], vreg[VLDS ? 1 : NKS];
  {
    const int keyc = min(key, S - 1);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const uint32_t off = (uint32_t)keyc * D + 16 * ks + 8 * hh;
      kreg[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(Kh + off));
      if constexpr (!VLDS) vreg[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(Vh + off));
    }
    // At D = 256 the kernel needs more than the 256 arch VGPRs.  K is read
    // only as an MFMA operand, which gfx950 takes from AGPRs, so its 64
    // registers are placed there once; otherwise the allocator moves values
    // between VGPRs and AGPRs on every tile.
    if constexpr (D == 256) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        u32x4 kk = __builtin_bit_cast(u32x4, kreg[ks]);
        asm volatile("" : "+a"(kk));
        kreg[ks] = __builtin_bit_cast(bf16x8, kk);
      }
    }
  }
  const uint16_t* Vw = nullptr;  // this wave's 32 rows of the V tile
  if constexpr (VLDS) Vw = sm.Vs + 32 * wave * D;

  f32x16 dk[NDO], dv[NDO];
#pragma unroll
  for (int db = 0; db < NDO; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }

  // This lane's dS write column: the even key of its lane pair, one row down
  // for the odd lane.
  const int dsw = (c32 & 1) * SRS + ((32 * wave + c32) & ~1);

  wait_vm_lds<0>();
  barrier_keep_loads();

  for (int qt = qt0; qt < nqt; ++qt) {
    const int buf = (qt - qt0) & 1;
    const int q0 = qt * BQ;
    if (qt + 1 < nqt) issue(qt + 1, buf ^ 1);  // buffer freed by the previous iteration
    __builtin_amdgcn_sched_barrier(0);

    const bool active = !CAUSAL || (q0 + BQ - 1 >= kw0);  // wave-uniform
    if (active) {
      const bool need_mask = (CAUSAL && q0 < kw0 + 31) || (kw0 + 32 > S) || (q0 + BQ > S);
      bwd_tile<D, Cfg, CAUSAL, WITH_DQ, VLDS, NDO>(sm, buf, of, kreg, vreg, Vw, dk, dv, q0, key, S, C, c32, hh, dsw,
                                                   need_mask);
    } else {
      if constexpr (WITH_DQ) {
#pragma unroll
        for (int r = 0; r < 2 * BQ / 4; r += 2) {
          const int row = 32 * (r >> 4) + 8 * ((r & 15) >> 2) + 4 * hh + (r & 3);
          *reinterpret_cast<uint32_t*>(&sm.dSs[row * SRS + dsw]) = 0u;
        }
      }
    }
    if constexpr (WITH_DQ) {
      __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (3 << 14));  // lgkmcnt(0): dS stores done
      barrier_keep_loads();  // dSs complete

    // ---- dQ[q, d] += scale * dS K over the workgroup's keys ---------------
#pragma unroll
    for (int j = 0; j < NDQ; ++j) {
      const int bi = wave * NDQ + j;
      const int qb = bi / NDB;
      const int db = bi % NDB;
      f32x16 acc0 = f32x16{}, acc1 = f32x16{};
#pragma unroll
      for (int t = 0; t < BK / 16; t += 2) {
        const int o0 = 16 * t * CPR * 8, o1 = 16 * (t + 1) * CPR * 8;
        acc0 = mfma32(lds_frag(&sm.dSs[(32 * qb + c32) * SRS + 16 * t + 8 * hh]),
                      tr_operand(at_bytes(sm.Ks, of.trk[db][0]) + o0, at_bytes(sm.Ks, of.trk[db][1]) + o0), acc0);
        acc1 = mfma32(lds_frag(&sm.dSs[(32 * qb + c32) * SRS + 16 * t + 16 + 8 * hh]),
                      tr_operand(at_bytes(sm.Ks, of.trk[db][0]) + o1, at_bytes(sm.Ks, of.trk[db][1]) + o1), acc1);
      }
      const uint32_t off0 = (uint32_t)(q0 + 32 * qb + 4 * hh) * D + 32 * db + c32;
      if (q0 + BQ <= S) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          unsafeAtomicAdd(dqh + off0 + (8 * (r >> 2) + (r & 3)) * D, (acc0[r] + acc1[r]) * scale);
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int q = q0 + 32 * qb + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (q < S) unsafeAtomicAdd(dqh + off0 + (8 * (r >> 2) + (r & 3)) * D, (acc0[r] + acc1[r]) * scale);
        }
      }
    }
    }  // WITH_DQ
    // next tile's loads landed (this wave's) and all LDS reads done; the
    // barrier publishes the tile and frees dSs
    __builtin_amdgcn_s_waitcnt((0) | (7 << 4) | (0 << 14));  // vmcnt(0) lgkmcnt(0)
    barrier_keep_loads();
  }

  // ---- epilogue: dK = scale * acc, dV = acc (bf16), staged in the query-tile
  // buffers (free once every wavefront is past the last tile) -----------------
  static_assert(2 * 32 * 32 * NDO <= 2 * Cfg::QTILE, "two staging slices per buffer pair");
  __builtin_amdgcn_s_waitcnt((0) | (7 << 4) | (0 << 14));  // vmcnt(0) lgkmcnt(0)
  __syncthreads();
  if (kw0 < S) {
    uint16_t* slice = (wave < 2 ? &sm.Qs[0][0] : &sm.dOs[0][0]) + (wave & 1) * 32 * 32 * NDO;
    store_dkdv_rows<NDO>(dk, dv, scale, slice, dK + base + (size_t)kw0 * D + d0, dV + base + (size_t)kw0 * D + d0, D,
                         S - kw0, lane);
  }
}

// dK/dV kernel of the split mode (D = 64 and 128; D = 256 with the columns
// split, below), and of the fused atomic mode at D = 128 with S a multiple
// of 128: the software-pipelined tile of dkdv_tile over 64-query tiles.  One workgroup
// of four wavefronts owns 128 keys; each
// wavefront keeps its 32 keys' K and V rows and dK, dV accumulators in
// registers.  The two query-tile buffers are separate __shared__ arrays and
// the loop is unrolled by two, so that every buffer a tile reads or loads
// into is known at compile time: the compiler then sees that the next tile's
// loads cannot alias this tile's LDS transpose reads and does not make those
// reads wait for the loads, which lets the loads be spread over the tile's
// MFMA work.
//
// Only unmasked tiles sit in the loop (two copies of the tile code, one per
// buffer set; four would not fit the register budget): a non-causal tile
// never needs the mask, also at lengths that are not a multiple of 128
// (query rows past S load as zeros and add nothing, keys past S reach only
// their own unstored dK / dV columns; see ntiles below), and a causal one
// only in the workgroup's first two query tiles (queries k0 .. k0 + 127,
// the diagonal block), which are peeled off before the loop.  (The atomic
// mode takes bwd_main_kernel at lengths that are not a multiple of 128.)
//
// DQ (the fused atomic mode): the kernel also forms dQ, so no second kernel
// recomputes S and dP.  Each tile's dS goes to LDS transposed (dS^T[key][q],
// two buffers); in the next tile's phase D every wavefront multiplies it, for
// its 32 columns of dQ, by the workgroup's 128 K rows (K^T fragments held in
// AGPRs since the start): dQ[q, 32 w + c] = sum_k dS[q, k] K[k, 32 w + c],
// 16 MFMAs per tile, and adds the 64 x 32 result, times scale, to the fp32
// accumulator in global memory with no-return buffer atomics (one workgroup
// per key tile, so each element of dQ receives one addition per key tile).
// The result is kept in registers over the barrier and its 32 atomics go
// out at the start of the following tile, so the end-of-tile wait for that
// tile's loads (the vector-memory counter does not order loads and stores)
// finds them long complete.  Non-causal workgroups start their walk over
// the query tiles at different tiles (rotated by key tile), so that the
// workgroups of one head running together add into different rows.
//
// D = 256 (DSPLIT = 2): the dK / dV columns are split between two workgroups
// per key tile (128 each, as in bwd_main_kernel at that head dim); each holds
// its keys' full K and V rows (the S and dP products contract over all 256
// columns) and recomputes P and dS.
template <int D, int DSPLIT, bool CAUSAL, bool DQ>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ nlse2, const float* __restrict__ delta,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, float* __restrict__ dq32, int BH, int S, float scale,
    float C) {
  static_assert((D == 128 && DSPLIT == 1) || (D == 64 && DSPLIT == 1 && !DQ) || (D == 256 && DSPLIT == 2 && !DQ),
                "D = 64 or 128, or D = 256 split in two");
  using Cfg = BwdCfg<D, 64>;
  constexpr int BK = Cfg::BK, BQ = Cfg::BQ, NKS = Cfg::NKS, NDB = Cfg::NDB, DMA_Q = Cfg::DMA_Q;
  constexpr int NDO = NDB / DSPLIT;  // output column blocks of this workgroup
  constexpr int NPIECE = 2 * DMA_Q + 1;  // Q pieces, dO pieces, then -LSE log2e / Delta
  static_assert(NPIECE == NKS + 1, "pieces are issued over phases A and B");
  // dS^T row stride (elements): 64 queries + 8, so that the rows of a
  // transpose read fall in distinct banks
  constexpr int DRS = BQ + 8;

  __shared__ __attribute__((aligned(1024))) uint16_t Qs0[Cfg::QTILE];
  __shared__ __attribute__((aligned(1024))) uint16_t Qs1[Cfg::QTILE];
  __shared__ __attribute__((aligned(1024))) uint16_t dOs0[Cfg::QTILE];
  __shared__ __attribute__((aligned(1024))) uint16_t dOs1[Cfg::QTILE];
  __shared__ __attribute__((aligned(256))) float nl0[Cfg::LROWS];
  __shared__ __attribute__((aligned(256))) float nl1[Cfg::LROWS];
  __shared__ __attribute__((aligned(256))) float dl0[Cfg::LROWS];
  __shared__ __attribute__((aligned(256))) float dl1[Cfg::LROWS];
  __shared__ __attribute__((aligned(256))) uint16_t dsT0[DQ ? BK * DRS : 8];
  __shared__ __attribute__((aligned(256))) uint16_t dsT1[DQ ? BK * DRS : 8];

  // one head's key tiles together on an XCD, except for causal passes with
  // fewer than 128 tiles per head, where the grid-wide heaviest-first order
  // balances the tail better (same-process A/B: non-causal 0.2-4 % faster,
  // ctx32k causal 3.7 % faster, S = 4096 / 8192 causal 2-3.5 % slower)
  int bh, kt2;
  const int ntl = gridDim.x / BH;
  xcd_head_order(blockIdx.x, BH, ntl, !CAUSAL || ntl >= 128, bh, kt2);
  const int ktile = kt2 / DSPLIT;  // causal: lowest keys (most work) first
  const int d0 = DSPLIT > 1 ? kt2 % DSPLIT * (D / DSPLIT) : 0;  // first dK / dV column
  const int k0 = ktile * BK;
  const size_t base = (size_t)bh * (size_t)S * D;
  const uint16_t* Qh = Q + base;
  const uint16_t* Kh = K + base;
  const uint16_t* Vh = V + base;
  const uint16_t* dOh = dO + base;
  const float* NLh = nlse2 + (size_t)bh * S;
  const float* DLh = delta + (size_t)bh * S;

  const int tid = threadIdx.x;
  // Wavefront index.  Read from the first lane (uniform by construction) it
  // makes the LDS-DMA destinations scalar values, which saves about 20
  // readfirstlanes per pair of tiles; the causal kernels keep the plain form,
  // with which their register allocation stays below the spill point.
  const int wave = CAUSAL ? (tid >> 6) : __builtin_amdgcn_readfirstlane(tid >> 6);
  // the index read from the first lane in every kernel, for the LDS-DMA
  // destinations (which must be uniform) only
  const int wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int hh = lane >> 5;
  const int c32 = lane & 31;
  const int kw0 = k0 + 32 * wave;
  const int key = kw0 + c32;

  BwdOffsets<D, Cfg> of;
  of.init(wave, lane, d0);
  // D = 256, non-causal: the Q / dO load offsets are formed per piece from
  // two per-lane values (dmaq_closed) instead of being held in eight
  // registers; held, they pushed this kernel into scratch, and every reload
  // of a spilled offset waited for all loads in flight (5 % of its time).
  // Made opaque once per tile below, so that the compiler does not hoist the
  // eight offsets back out of the loop.  (The causal kernel does not spill,
  // and measured 1 % slower this way.)
  constexpr bool DMA_CLOSED = D == 256 && !CAUSAL;
  uint32_t dmx = 0, dmy = 0;
  if constexpr (DMA_CLOSED) {
    const int lr = lane / (D / 8), cc = lane % (D / 8);
    dmx = (uint32_t)(cc ^ (4 * lr));
    dmy = (uint32_t)(32 * D * wave_u + 2 * D * lr);
  }

  // query tiles in walking order: causal from the diagonal on, non-causal
  // (fused mode) rotated by key tile
  const int nqt = (S + BQ - 1) / BQ;
  const int qt0 = CAUSAL ? (k0 / BQ) : 0;
  // Any S: the tile count is rounded up to even (the loop takes tiles in
  // pairs; the atomic mode's lengths, multiples of 128, give an even count).  A tile past the last one, like the rows
  // past S of a partial one, loads as zeros (out-of-range lanes of the
  // range-checked LDS-direct loads write zeros), and a zero query row adds
  // nothing: its Q, dO, -LSE log2e and Delta are 0, so P = 1, dP = 0 and
  // dS = 0, while dO = 0 zeroes its dV term.  Keys past S are clamped to
  // S - 1 and only their own (unstored) dK / dV columns see them.
  const int ntiles = (nqt - qt0 + 1) & ~1;
  const int rot = (!CAUSAL && DQ) ? (ktile * (nqt >= 8 ? nqt / 8 : 1)) % nqt : 0;
  auto qt_at = [&](int i) { return CAUSAL ? qt0 + i : !DQ ? i : (i + rot < nqt ? i + rot : i + rot - nqt); };

  // piece p of query tile qt's loads into buffer set P (0: Qs0 ..., 1: Qs1 ...)
  auto piece = [&](int qt, auto P, int p) {
    constexpr int set = decltype(P)::value;
    uint16_t* qd = set ? Qs1 : Qs0;
    uint16_t* dd = set ? dOs1 : dOs0;
    const int q0 = qt * BQ;
    if (p < DMA_Q) {
      if constexpr (DMA_CLOSED)
        dma_row_at<D, DMA_Q>(Qh, q0, S, qd, wave_u, p, dmaq_closed<D>(dmx, dmy, p));
      else
        dma_row_part<D, DMA_Q, false>(Qh, q0, BQ, S, qd, wave_u, of.dmaq, p);
    } else if (p < 2 * DMA_Q) {
      if constexpr (DMA_CLOSED)
        dma_row_at<D, DMA_Q>(dOh, q0, S, dd, wave_u, p - DMA_Q, dmaq_closed<D>(dmx, dmy, p - DMA_Q));
      else
        dma_row_part<D, DMA_Q, false>(dOh, q0, BQ, S, dd, wave_u, of.dmaq, p - DMA_Q);
    } else if (p == 2 * DMA_Q) {
      // -LSE log2e rows from waves 0 and 2, Delta from 1 and 3 (the pairs
      // write the same values): no branch on the wavefront index, which
      // would split the tile into blocks the compiler moves the softmax
      // across
      const bool odd = (wave_u & 1) != 0;
      const float* src = odd ? DLh : NLh;
      float* dst = odd ? (set ? dl1 : dl0) : (set ? nl1 : nl0);
      // rows past S load as zeros (range-checked)
      lds_dma<4>(src, (uint32_t)S * 4u, (uint32_t)(q0 + lane) * 4u, dst);
    }
  };

#pragma unroll
  for (int p = 0; p < NPIECE; ++p) piece(qt_at(0), std::integral_constant<int, 0>{}, p);

  // K / V rows of this lane's key as MFMA operands (rows past the end are
  // clamped; their P is masked).  The pipelined tile needs more than the 256
  // arch VGPRs; K and V are read only as MFMA operands, which gfx950 takes
  // from AGPRs, so they are placed there once instead of being spilled and
  // reloaded.  V is held negated (a sign flip, exact in bf16): the dP
  // accumulator starts from Delta, so the MFMAs leave Delta - dP in it and
  // dS = -P (Delta - dP) needs no subtraction per element.
  bf16x8 kreg[NKS], vreg[NKS];
  {
    const int keyc = min(key, S - 1);
    u32x4 kk[NKS], vv[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const uint32_t off = (uint32_t)keyc * D + 16 * ks + 8 * hh;
      kk[ks] = *reinterpret_cast<const u32x4*>(Kh + off);
      vv[ks] = *reinterpret_cast<const u32x4*>(Vh + off) ^ 0x80008000u;
    }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      asm volatile("" : "+a"(kk[ks]), "+a"(vv[ks]));
      kreg[ks] = __builtin_bit_cast(bf16x8, kk[ks]);
      vreg[ks] = __builtin_bit_cast(bf16x8, vv[ks]);
    }
  }

  // ---- fused dQ: operands, offsets, the atomic target ---------------------
  // B operand of k-step t: K[k0 + 16 t + slot key][32 wave + c32] with slot j
  // of lane half hh holding key 8 (j / 4) + 4 hh + j % 4 (the key order of the
  // dS^T transpose reads); keys past S are zero.
  bf16x8 kT[DQ ? 8 : 1];
  // A operand reads: dS^T rows (keys) 16 t + 8 r2 + 4 hh + (i >> 2), columns
  // (queries) 32 qb + 16 (g16 & 1) + 4 (i & 3): byte offsets for r2 = 0, 1
  int dso[2] = {0, 0};
  int dsw = 0;  // this lane's dS^T row (its key) in bytes
  // the head's fp32 dQ rows as a buffer resource: rows past S fall outside
  // it, so the atomics of a ragged tile's missing rows are dropped
  const __amdgpu_buffer_rsrc_t dqrs = __builtin_amdgcn_make_buffer_rsrc(
      DQ ? (void*)(dq32 + (size_t)bh * S * D) : (void*)dq32, (short)0, DQ ? S * D * 4 : 0, kBufRsrcWord3);
  uint32_t dqlane = 0;  // byte offset of this lane's dQ element in row 0 of a 4-row group
  if constexpr (DQ) {
    const int i16 = lane & 15, g16 = lane >> 4;
#pragma unroll
    for (int r2 = 0; r2 < 2; ++r2)
      dso[r2] = ((8 * r2 + 4 * (g16 >> 1) + (i16 >> 2)) * DRS + 16 * (g16 & 1) + 4 * (i16 & 3)) * 2;
    dsw = (32 * wave + c32) * DRS * 2;
    const int dcol = 32 * wave + c32;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      uint32_t w[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        uint16_t h2[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int j = 2 * m + u;
          const int kk = k0 + 16 * t + 8 * (j >> 2) + 4 * hh + (j & 3);
          h2[u] = kk < S ? Kh[(size_t)kk * D + dcol] : (uint16_t)0;
        }
        w[m] = (uint32_t)h2[0] | ((uint32_t)h2[1] << 16);
      }
      u32x4 v = {w[0], w[1], w[2], w[3]};
      asm volatile("" : "+a"(v));
      kT[t] = __builtin_bit_cast(bf16x8, v);
    }
    dqlane = (uint32_t)((4 * hh) * D + dcol) * 4u;
  }

  f32x16 dk[NDO], dv[NDO];
#pragma unroll
  for (int db = 0; db < NDO; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }
  wait_vm_lds<0>();
  barrier_keep_loads();

  // dQ of a finished tile (its dS^T in `src`, queries q0 ..): per k-step t,
  // the A operands of both 32-query blocks by transpose reads, two MFMAs;
  // then the atomics (scale applied).
  auto dq_read = [&](const uint16_t* src, int t, int qb) {
    const int o = (16 * t * DRS + 32 * qb) * 2;
    return tr_operand(at_bytes(src, dso[0] + o), at_bytes(src, dso[1] + o));
  };
  auto dq_atomics = [&](const f32x16 (&acc)[2], int q0) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t voff = dqlane + (uint32_t)((q0 + 32 * qb + 8 * g) * D) * 4u;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(acc[qb][4 * g + e] * scale, dqrs, voff + e * D * 4, 0, 0);
      }
    }
  };

  // Hooks for dkdv_tile in the fused mode: this tile's dS^T into `cur`, the
  // previous tile's dQ from `prev` in phase D.
  struct Hooks {
    uint16_t* cur;
    const uint16_t* prev;
    int dsw, hh;
    const int* dso;
    const bf16x8* kT;
    f32x16 acc[2];
    bf16x8 a[2][2];  // [parity of k-step][qb]
    int DRS_;
    __device__ __forceinline__ bf16x8 rd(int t, int qb) {
      const int o = (16 * t * DRS_ + 32 * qb) * 2;
      return tr_operand(at_bytes(prev, dso[0] + o), at_bytes(prev, dso[1] + o));
    }
    __device__ __forceinline__ void store(int qb, const bf16x8 (&d)[2]) {
      // register 8 h2 + e4 (h2 = 0, 1) of pair half holds query 32 qb + 8 (2 half + h2) + 4 hh + e4:
      // four consecutive queries per 8-byte store
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const u32x4 w = __builtin_bit_cast(u32x4, d[half]);
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int col = 32 * qb + 8 * (2 * half + h2) + 4 * hh;
          *reinterpret_cast<u32x2*>(reinterpret_cast<char*>(cur) + dsw + col * 2) = u32x2{w[2 * h2], w[2 * h2 + 1]};
        }
      }
    }
    __device__ __forceinline__ void step(int i) {
      if (i == 0) {
        acc[0] = f32x16{};
        acc[1] = f32x16{};
        a[0][0] = rd(0, 0);
        a[0][1] = rd(0, 1);
      }
      if (i + 1 < 8) {
        a[(i + 1) & 1][0] = rd(i + 1, 0);
        a[(i + 1) & 1][1] = rd(i + 1, 1);
      }
      acc[0] = mfma32(a[i & 1][0], kT[i], acc[0]);
      acc[1] = mfma32(a[i & 1][1], kT[i], acc[1]);
    }
  };

  // dQ of tile i - 1, formed during tile i, waiting for its atomics
  f32x16 pend[2] = {f32x16{}, f32x16{}};

  // one tile: reads buffer set P, loads the next tile into set 1 - P.  M:
  // masked tile (the causal diagonal block), where a causal wave may also have no
  // query at or after its keys (inactive: it only issues its loads; in the
  // fused mode every wave stays active, its masked dS being the zeros the
  // dQ product needs).
  auto tile = [&](int i, auto P, auto M) {
    constexpr int set = decltype(P)::value;
    constexpr bool MASK = decltype(M)::value;
    using Next = std::integral_constant<int, 1 - set>;
    const int qt = qt_at(i);
    const int q0 = qt * BQ;
    const bool has_next = i + 1 < ntiles;
    const int qtn = has_next ? qt_at(i + 1) : qt;
    const bool active = DQ || !(CAUSAL && MASK) || (q0 + BQ - 1 >= kw0);  // wave-uniform
    if constexpr (DQ) {
      if (i >= 2) dq_atomics(pend, qt_at(i - 2) * BQ);  // formed during the previous tile
    }
    if (active) {
      // after the last tile the pieces reload it into the free set (in bounds,
      // never read), which keeps the tile branch-free
      auto part = [&](int p) {
        if (p < NPIECE) piece(qtn, Next{}, p);
      };
      const uint16_t* Qb = set ? Qs1 : Qs0;
      const uint16_t* dOb = set ? dOs1 : dOs0;
      const float* nl = set ? nl1 : nl0;
      const float* dl = set ? dl1 : dl0;
      // The read offsets are made opaque per tile: otherwise each buffer set's
      // full addresses are loop-invariant, get hoisted and held in registers
      // (twice the offsets); this way every read is offset register + the
      // array's constant LDS address, which folds into the instruction.
      BwdOffsets<D, Cfg> ot = of;
      if constexpr (DMA_CLOSED) asm volatile("" : "+v"(dmx), "+v"(dmy));
      // D = 256: the swizzle XORs only the low four bits of a chunk index, so
      // the offsets of reduction steps 8 .. 15 are those of steps 0 .. 7 plus
      // 256 bytes; written after the opaque copies, the constant folds into
      // the LDS instructions' immediate offset (eight registers fewer)
      constexpr int NOPQ = D == 256 ? NKS / 2 : NKS;
#pragma unroll
      for (int ks = 0; ks < NOPQ; ++ks) asm volatile("" : "+v"(ot.arow[ks]));
#pragma unroll
      for (int ks = NOPQ; ks < NKS; ++ks) ot.arow[ks] = ot.arow[ks - NOPQ] + 256;
#pragma unroll
      for (int db = 0; db < NDO; ++db) asm volatile("" : "+v"(ot.trq[db][0]), "+v"(ot.trq[db][1]));
      if constexpr (DQ) {
        int dso_t[2] = {dso[0], dso[1]};
        int dsw_t = dsw;
        asm volatile("" : "+v"(dso_t[0]), "+v"(dso_t[1]), "+v"(dsw_t));
        Hooks hk{set ? dsT1 : dsT0, set ? dsT0 : dsT1, dsw_t, hh, dso_t, kT, {}, {}, DRS};
        dkdv_tile<D, Cfg, CAUSAL, MASK>(Qb, dOb, nl, dl, ot, kreg, vreg, dk, dv, q0, key, S, C, hh, part, hk);
        // the previous tile's dQ (a first tile has none: its MFMAs read a
        // buffer no tile has written yet, and the result is never added)
        pend[0] = hk.acc[0];
        pend[1] = hk.acc[1];
      } else {
        dkdv_tile<D, Cfg, CAUSAL, MASK>(Qb, dOb, nl, dl, ot, kreg, vreg, dk, dv, q0, key, S, C, hh, part);
      }
    } else if (has_next) {
#pragma unroll
      for (int p = 0; p < NPIECE; ++p) piece(qtn, Next{}, p);
    }
    // the next tile's loads landed (this wave's) and all LDS reads and dS
    // stores done; the barrier publishes the tile and frees this one
    __builtin_amdgcn_s_waitcnt((0) | (7 << 4) | (0 << 14));  // vmcnt(0) lgkmcnt(0)
    barrier_keep_loads();
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  using M = std::false_type;
  int i = 0;
  if constexpr (CAUSAL) {  // diagonal block: qt0 even, ntiles >= 2
    tile(0, P0{}, std::true_type{});
    tile(1, P1{}, std::true_type{});
    i = 2;
  }
  for (; i < ntiles; i += 2) {
    tile(i, P0{}, M{});
    tile(i + 1, P1{}, M{});
  }

  // ---- fused: the last two tiles' dQ --------------------------------------
  if constexpr (DQ) {
    if (ntiles >= 2) dq_atomics(pend, qt_at(ntiles - 2) * BQ);
    const int last = ntiles - 1;
    const uint16_t* src = (last & 1) ? dsT1 : dsT0;
    f32x16 acc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      acc[0] = mfma32(dq_read(src, t, 0), kT[t], acc[0]);
      acc[1] = mfma32(dq_read(src, t, 1), kT[t], acc[1]);
    }
    dq_atomics(acc, qt_at(last) * BQ);
  }

  // ---- epilogue: dK = scale * acc, dV = acc (bf16), staged in the query-tile
  // buffers (free once every wavefront is past the last tile) --------------
  static_assert(2 * 32 * 32 * NDO <= Cfg::QTILE, "two staging slices per buffer");
  __builtin_amdgcn_s_waitcnt((0) | (7 << 4) | (0 << 14));  // vmcnt(0) lgkmcnt(0)
  __syncthreads();
  uint16_t* slice = (wave < 2 ? Qs0 : Qs1) + (wave & 1) * 32 * 32 * NDO;
  store_dkdv_rows<NDO>(dk, dv, scale, slice, dK + base + (size_t)kw0 * D + d0, dV + base + (size_t)kw0 * D + d0, D,
                       S - kw0, lane);
}

template <bool CAUSAL, bool DQ, int D = 128, int DSPLIT = 1>
static hipError_t launch_dkdv_pipe_rt(const BwdArgs& a, hipStream_t st) {
  const int BH = a.B * a.H;
  const int nkt = (a.S + 127) / 128;
  const int kid = DQ ? KID_BWD_MAIN : KID_BWD_DKDV;
  prof_begin(kid, st);
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, DSPLIT, CAUSAL, DQ>), dim3(nkt * BH * DSPLIT), dim3(256), 0, st,
                     (const uint16_t*)a.Q,
                     (const uint16_t*)a.K, (const uint16_t*)a.V, (const uint16_t*)a.dO, a.nlse2, a.delta,
                     (uint16_t*)a.dK, (uint16_t*)a.dV, a.dq32, BH, a.S, a.scale, a.scale * kLog2e);
  prof_end(kid, st);
  return hipGetLastError();
}

template <bool CAUSAL>
static hipError_t launch_dkdv_pipe_t(const BwdArgs& a, hipStream_t st) {
  return launch_dkdv_pipe_rt<CAUSAL, false>(a, st);
}

// Delta_i = sum_d dO_id O_id (fp32), nlse2_i = -LSE_i log2(e), and zero the
// fp32 dQ accumulator (atomic mode).  D/8 lanes share one row; each lane
// takes eight columns.
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const uint16_t* __restrict__ O,
                                                      const uint16_t* __restrict__ dO,
                                                      const float* __restrict__ LSE,
                                                      float* __restrict__ delta, float* __restrict__ nlse2,
                                                      float* __restrict__ dq32, long rows) {
  constexpr int LPR = D / 8;
  const long row = ((long)blockIdx.x * 256 + threadIdx.x) / LPR;
  const int c = threadIdx.x % LPR;
  float acc = 0.0f;
  if (row < rows) {
    const u32x4 o = *reinterpret_cast<const u32x4*>(O + row * D + 8 * c);
    const u32x4 g = *reinterpret_cast<const u32x4*>(dO + row * D + 8 * c);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      acc = __builtin_fmaf(__uint_as_float(o[m] << 16), __uint_as_float(g[m] << 16), acc);
      acc = __builtin_fmaf(__uint_as_float(o[m] & 0xffff0000u), __uint_as_float(g[m] & 0xffff0000u), acc);
    }
    if (dq32 != nullptr) {
      f32x4* z = reinterpret_cast<f32x4*>(dq32 + row * D + 8 * c);
      z[0] = f32x4{};
      z[1] = f32x4{};
    }
  }
#pragma unroll
  for (int off = LPR / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if (c == 0 && row < rows) {
    delta[row] = acc;
    nlse2[row] = -LSE[row] * kLog2e;
  }
}

// dQ (bf16) from the fp32 accumulator, eight elements per thread.
__global__ __launch_bounds__(256) void dq_convert_kernel(const float* __restrict__ dq32,
                                                         uint16_t* __restrict__ dQ, long n8) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i < n8) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(dq32 + 8 * i);
    const f32x4 b = *reinterpret_cast<const f32x4*>(dq32 + 8 * i + 4);
    *reinterpret_cast<u32x4*>(dQ + 8 * i) =
        __builtin_bit_cast(u32x4, to_bf16x8(a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]));
  }
}

// The atomic mode keeps full-width dK, dV and the dQ tile's K operands in
// one workgroup, which does not fit at D = 256; the split mode divides the
// dK / dV columns there.
bool bwd_supported(int D, bool atomic) { return D == 64 || D == 128 || (D == 256 && !atomic); }

template <int D, int BQ, bool CAUSAL, bool WITH_DQ, bool VLDS, int OCC, int DSPLIT = 1, bool RAGGED = true>
static hipError_t launch_main_t(const BwdArgs& a, hipStream_t st) {
  const int BH = a.B * a.H;
  const int nkt = (a.S + BwdCfg<D, BQ>::BK - 1) / BwdCfg<D, BQ>::BK;
  const int kid = WITH_DQ ? KID_BWD_MAIN : KID_BWD_DKDV;
  prof_begin(kid, st);
  hipLaunchKernelGGL((bwd_main_kernel<D, BQ, CAUSAL, WITH_DQ, VLDS, OCC, DSPLIT, RAGGED>), dim3(nkt * BH * DSPLIT),
                     dim3(256),
                     0, st,
                     (const uint16_t*)a.Q, (const uint16_t*)a.K, (const uint16_t*)a.V,
                     (const uint16_t*)a.dO, a.nlse2, a.delta, a.dq32, (uint16_t*)a.dK,
                     (uint16_t*)a.dV, BH, a.S, a.scale, a.scale * kLog2e);
  prof_end(kid, st);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_pre_t(const BwdArgs& a, hipStream_t st) {
  const long rows = (long)a.B * a.H * a.S;
  const long threads = rows * (D / 8);
  prof_begin(KID_BWD_PRE, st);
  hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st,
                     (const uint16_t*)a.O, (const uint16_t*)a.dO, a.LSE, a.delta, a.nlse2, a.dq32, rows);
  prof_end(KID_BWD_PRE, st);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
static hipError_t launch_dkdv_t(const BwdArgs& a, hipStream_t st) {
  if constexpr (D == 128) {
    return launch_dkdv_pipe_t<CAUSAL>(a, st);
  } else if constexpr (D == 256) {
    // each workgroup forms 128 of the 256 columns: the pipelined 64-query
    // tile (variant 1: the one-pass tile over 32-query tiles with the V tile
    // in LDS)
    if (kernel_variant(VAR_DKDV) != 1) return launch_dkdv_pipe_rt<CAUSAL, false, D, 2>(a, st);
    return (a.S % 32 == 0) ? launch_main_t<D, 32, CAUSAL, false, true, 1, 2, false>(a, st)
                           : launch_main_t<D, 32, CAUSAL, false, true, 1, 2, true>(a, st);
  } else {
    // the pipelined tile (variant 1: the one-pass tile)
    if (kernel_variant(VAR_DKDV) != 1) return launch_dkdv_pipe_rt<CAUSAL, false, D, 1>(a, st);
    return launch_main_t<D, 32, CAUSAL, false, false, 2>(a, st);
  }
}

template <bool WITH_DQ>
static hipError_t launch_main(const BwdArgs& a, hipStream_t st) {
  if constexpr (WITH_DQ) {
    switch (a.D * 2 + (a.causal ? 1 : 0)) {
      case 128: return launch_main_t<64, 64, false, true, false, 1>(a, st);
      case 129: return launch_main_t<64, 64, true, true, false, 1>(a, st);
      // S a multiple of 128: the fused pipelined kernel; otherwise the
      // one-pass tile (the fused tile's masked-on-every-tile form needs more
      // registers than the compiler can allocate)
      case 256:
        return a.S % 128 == 0 ? launch_dkdv_pipe_rt<false, true>(a, st)
                              : launch_main_t<128, 64, false, true, false, 1>(a, st);
      case 257:
        return a.S % 128 == 0 ? launch_dkdv_pipe_rt<true, true>(a, st)
                              : launch_main_t<128, 64, true, true, false, 1>(a, st);
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (a.D * 2 + (a.causal ? 1 : 0)) {
      case 128: return launch_dkdv_t<64, false>(a, st);
      case 129: return launch_dkdv_t<64, true>(a, st);
      case 256: return launch_dkdv_t<128, false>(a, st);
      case 257: return launch_dkdv_t<128, true>(a, st);
      case 512: return launch_dkdv_t<256, false>(a, st);
      case 513: return launch_dkdv_t<256, true>(a, st);
      default: return hipErrorInvalidValue;
    }
  }
}

static hipError_t launch_pre(const BwdArgs& a, hipStream_t st) {
  switch (a.D) {
    case 64: return launch_pre_t<64>(a, st);
    case 128: return launch_pre_t<128>(a, st);
    case 256: return launch_pre_t<256>(a, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_atomic(const BwdArgs& a, hipStream_t st) {
  hipError_t e = launch_pre(a, st);
  if (e != hipSuccess) return e;
  e = launch_main<true>(a, st);
  if (e != hipSuccess) return e;
  const long n8 = (long)a.B * a.H * a.S * a.D / 8;
  prof_begin(KID_DQ_CONVERT, st);
  hipLaunchKernelGGL(dq_convert_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st,
                     (const float*)a.dq32, (uint16_t*)a.dQ, n8);
  prof_end(KID_DQ_CONVERT, st);
  return hipGetLastError();
}

// Split mode: the dQ kernel forms Delta and -LSE log2e of its rows (it
// holds their dO anyway) and writes them for the dK/dV kernel that follows,
// so no separate preprocessing pass runs.
hipError_t launch_bwd_split(const BwdArgs& a, hipStream_t st) {
  BwdArgs b = a;
  b.dq32 = nullptr;
  hipError_t e = launch_bwd_dq(b, st);
  if (e != hipSuccess) return e;
  return launch_main<false>(b, st);
}

}  // namespace attn97

// kv_stream.hpp - streaming K/V (or any [S, D] bf16 matrix) tiles through
// swizzled LDS buffers with LDS-direct buffer loads, and the per-lane LDS offsets of
// the MFMA operands read from those tiles.  Used by the forward kernel and
// by the dQ kernel of the split backward pass, which walk the key sequence
// the same way.
#pragma once

#include "device_common.hpp"
#include "tile_layout.hpp"

namespace attn97 {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Tile configuration: head dim D, BC keys per tile, NW wavefronts (32 query
// rows each) per workgroup, NBUF LDS buffers per K and V tile.  With three
// buffers, loads are issued two iterations before they are consumed and a
// wave only waits for the ones issued an iteration earlier.
template <int D_, int BC_, int NW_, int NBUF_>
struct FwdCfg {
  static constexpr int D = D_;
  static constexpr int BC = BC_;                       // keys per tile
  static constexpr int NW = NW_;                       // wavefronts per workgroup
  static constexpr int NBUF = NBUF_;                   // LDS buffers per tile kind
  static constexpr int BR = 32 * NW;                   // queries per workgroup
  static constexpr int CPR = D / 8;                    // 16-byte chunks per row
  static constexpr int TILE_BYTES = BC * D * 2;
  static constexpr int NKB = BC / 32;                  // 32-key blocks per tile
  static constexpr int NKS = D / 16;                   // reduction steps over D
  static constexpr int NDB = D / 32;                   // 32-wide blocks of D
  static constexpr int DMA_PER_WAVE = TILE_BYTES / 1024 / NW;  // 1 KiB loads per wave per tile
  static constexpr int LDS_BYTES = 2 * NBUF * TILE_BYTES;
  static_assert(DMA_PER_WAVE >= 1 && DMA_PER_WAVE * 1024 * NW == TILE_BYTES, "tile split over waves");
  static_assert(NBUF == 2 || NBUF == 3, "two or three buffers");
  static_assert(BC % 32 == 0 && BC >= 32, "key tile");
};

// Issue this wave's share of one tile load (rows k0.. of a [S, D] bf16
// matrix, k0 < S) into the swizzled LDS tile `dst`: lane l of load n fills physical
// chunk 64 * (wave * DMA_PER_WAVE + n) + l.  `loff[n]` is that chunk's
// logical element offset inside the tile (row * D + 8 * chunk), fixed per
// lane.  The buffer resource ends at row S, so in a ragged last tile the rows
// past S read as zero (a range-checked buffer load returns zero and the LDS
// copy stores it); the scores of those keys are masked, and zero V rows
// contribute nothing.  No per-tile offset arithmetic is needed.
// dma_tile_part issues only this wave's n-th 1 KiB piece: a kernel can spread
// a tile's pieces over its MFMA work (issued back to back they fill the
// memory pipeline and stall the wavefront).
template <class Cfg>
__device__ __forceinline__ void dma_tile_part(const uint16_t* __restrict__ src, int k0, int S, uint16_t* dst,
                                              int wave, const uint32_t (&loff)[Cfg::DMA_PER_WAVE], int n) {
  constexpr int NPW = Cfg::DMA_PER_WAVE, D = Cfg::D;
  const uint16_t* tile = src + (size_t)k0 * D;
  lds_dma<16>(tile, (uint32_t)(S - k0) * (uint32_t)(D * 2), loff[n] * 2, dst + 512 * (wave * NPW + n));
}

template <class Cfg>
__device__ __forceinline__ void dma_tile(const uint16_t* __restrict__ src, int k0, int S, uint16_t* dst,
                                         int wave, const uint32_t (&loff)[Cfg::DMA_PER_WAVE]) {
#pragma unroll
  for (int n = 0; n < Cfg::DMA_PER_WAVE; ++n) dma_tile_part<Cfg>(src, k0, S, dst, wave, loff, n);
}

// Round eight probabilities to bf16 as four packed 32-bit words for the MFMA
// operand.  The words are formed as 32-bit scalars: reading 32-bit words
// back out of a bf16 vector made hipcc reuse one word for all four.  (The
// row sum is taken from the fp32 values: summing the bf16-rounded ones would
// put a 2^-9 relative error into the log-sum-exp.)
__device__ __forceinline__ bf16x8 pack_probs(const float (&p)[8]) {
  u32x4 w;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    const f32x2 v = {p[2 * m], p[2 * m + 1]};
    w[m] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  }
  return as_bf16x8(w);
}

// Per-lane LDS offsets (elements) that stay fixed over the whole loop.
template <class Cfg>
struct FwdOffsets {
  static constexpr int D = Cfg::D, NKS = Cfg::NKS, NDB = Cfg::NDB, CPR = Cfg::CPR;
  // K operand: row c32 (+32 kb), chunk 2 ks + hh.  The swizzle depends on
  // row & 15 only, so the key block adds 32 * CPR chunks.
  int kfrag[NKS];
  // V^T operand: rows 8 r2 + 4 h + (i >> 2) (+16 t), column 32 db + 16 (g & 1)
  // + 4 (i & 3); the key group adds 16 * CPR chunks.
  int vfrag[NDB][2];
  // DMA source offsets of this lane's chunks.
  uint32_t dma[Cfg::DMA_PER_WAVE];

  __device__ __forceinline__ void init(int wave, int lane) {
    const int hh = lane >> 5, c32 = lane & 31, i = lane & 15, g16 = lane >> 4;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) kfrag[ks] = swz_chunk<D>(c32, 2 * ks + hh) * 8;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int d = 32 * db + 16 * (g16 & 1) + 4 * (i & 3);
#pragma unroll
      for (int r2 = 0; r2 < 2; ++r2)
        vfrag[db][r2] = swz_chunk<D>(8 * r2 + 4 * (g16 >> 1) + (i >> 2), d >> 3) * 8 + (d & 7);
    }
    if constexpr (D == 256) {
      // The swizzle XORs only the low four bits of the chunk index, so chunks
      // 16 apart sit 128 elements apart in every row: the upper half's
      // offsets are written as the lower half's plus a constant, which folds
      // into the LDS instructions' immediate offset and halves the registers
      // that hold offsets (the D = 256 tiles are short of arch VGPRs).
#pragma unroll
      for (int ks = NKS / 2; ks < NKS; ++ks) kfrag[ks] = kfrag[ks - NKS / 2] + 128;
#pragma unroll
      for (int db = NDB / 2; db < NDB; ++db)
#pragma unroll
        for (int r2 = 0; r2 < 2; ++r2) vfrag[db][r2] = vfrag[db - NDB / 2][r2] + 128;
    }
#pragma unroll
    for (int n = 0; n < Cfg::DMA_PER_WAVE; ++n) {
      int row, c;
      unswz_chunk<D>(64 * (wave * Cfg::DMA_PER_WAVE + n) + lane, row, c);
      dma[n] = (uint32_t)(row * D + 8 * c);
    }
  }
};

}  // namespace attn97

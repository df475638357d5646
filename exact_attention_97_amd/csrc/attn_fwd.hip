// attn_fwd.hip - forward pass of exact attention on gfx950.
//
// One workgroup of four wavefronts owns a tile of 128 query rows of one
// (batch, head); each wavefront owns 32 of those rows and walks the key/value
// sequence one tile of BC keys at a time:
//
//   S^T = K Q^T          bf16 MFMA, fp32 accumulate (scores, keys x queries)
//   mask, row max        in-lane over the wavefront's half, one swap of halves
//   conditional rescale  only when some row's max grew by more than tau (log2)
//   P = exp2(S*c - m)    native v_exp_f32 or the FMA-pipe polynomial
//   O^T += V^T P^T       bf16 MFMA with P taken straight from registers
//
// followed by O = O / l and LSE = ln2 * (m + log2 l).  The two matrix
// products are the ones attention is made of (page "FlashAttention-4 : comment
// Together AI a accéléré l'attention sur GPU Blackwell", section "Pourquoi
// l'approche standard ne fonctionne plus"); the software exponential and the
// conditional rescaling follow the abstract of "FlashAttention-4: Algorithm
// and Kernel Pipelining Co-Design for Asymmetric Hardware Scaling", and the
// overlap of the matrix products with the softmax of another block follows
// page "FlashAttention-3 и FlashAttention-4", section "Чередование matmul и
// softmax".
//
// Layout choices:
// * S is computed transposed (keys as MFMA rows, queries as columns), so all
//   scores of one query row sit in one lane pair (l, l+32): the row max and
//   row sum are in-lane and the rescale of the output accumulator is a
//   per-lane scalar.
// * K and V tiles go from HBM straight into LDS with global_load_lds (16
//   bytes per lane, no register staging), row-major with an XOR swizzle of
//   the 16-byte chunks chosen so that both the K operand reads
//   (ds_read_b128, 16 rows at one chunk) and the V operand reads
//   (ds_read_b64_tr_b16, 4 rows x 32 bytes) hit distinct banks.
// * V^T is read with the LDS transpose load: each lane gathers four keys at
//   its own d column, which is exactly the V^T MFMA operand.
//
// Pipeline: while the softmax of tile j runs on the VALU, the MFMA unit
// computes the scores of tile j+1; then P_j V_j.  K tiles are loaded two
// tiles ahead and V tiles one ahead, each into a double buffer, so one
// barrier per tile suffices.
#include "attn_kernels.hpp"
#include "device_common.hpp"

namespace attn97 {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

template <int D>
struct FwdCfg {
  static constexpr int BC = (D == 64) ? 128 : (D == 128 ? 64 : 32);  // keys per tile
  static constexpr int BR = 128;                                     // queries per workgroup
  static constexpr int CPR = D / 8;                                  // 16-byte chunks per row
  static constexpr int TILE_BYTES = BC * D * 2;                      // 16 KiB
  static constexpr int NKB = BC / 32;                                // 32-key blocks per tile
  static constexpr int NKS = D / 16;                                 // reduction steps over D
  static constexpr int NDB = D / 32;                                 // 32-wide blocks of D
  static constexpr int DMA_PER_WAVE = TILE_BYTES / 1024 / 4;         // 1 KiB loads per wave per tile
  static_assert(TILE_BYTES == 16384, "tile size");
};

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

// Issue this wave's share of one tile load (rows k0.. of a [S, D] bf16
// matrix) into the swizzled LDS tile `dst`: lane l of load n fills physical
// chunk 64 * (wave * DMA_PER_WAVE + n) + l.  `loff[n]` is that chunk's
// logical element offset inside the tile (row * D + 8 * chunk), fixed per
// lane.  In a ragged last tile, rows past S are clamped to S-1 (finite data;
// the scores of those keys are masked).
template <int D>
__device__ __forceinline__ void dma_tile(const uint16_t* __restrict__ src, int k0, int S, uint16_t* dst,
                                         int wave, const uint32_t (&loff)[FwdCfg<D>::DMA_PER_WAVE]) {
  constexpr int NPW = FwdCfg<D>::DMA_PER_WAVE, BC = FwdCfg<D>::BC;
  const uint16_t* tile = src + (size_t)k0 * D;
  const bool ragged = k0 + BC > S;
#pragma unroll
  for (int n = 0; n < NPW; ++n) {
    uint32_t off = loff[n];
    if (ragged) {
      const uint32_t row = off / D;
      const uint32_t last = (uint32_t)(S - 1 - k0);
      off = (row > last ? last : row) * D + off % D;
    }
    __builtin_amdgcn_global_load_lds(tile + off, (__attribute__((address_space(3))) void*)(dst + 512 * (wave * NPW + n)),
                                     16, 0, 0);
  }
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
template <int D>
struct FwdOffsets {
  using Cfg = FwdCfg<D>;
  static constexpr int NKS = Cfg::NKS, NDB = Cfg::NDB, CPR = Cfg::CPR;
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
#pragma unroll
    for (int n = 0; n < Cfg::DMA_PER_WAVE; ++n) {
      int row, c;
      unswz_chunk<D>(64 * (wave * Cfg::DMA_PER_WAVE + n) + lane, row, c);
      dma[n] = (uint32_t)(row * D + 8 * c);
    }
  }
};

template <int D, int EXPMODE>
struct FwdWave {
  using Cfg = FwdCfg<D>;
  static constexpr int NKB = Cfg::NKB, NKS = Cfg::NKS, NDB = Cfg::NDB, BC = Cfg::BC, CPR = Cfg::CPR;

  // S^T of one tile: sacc[kb] = K[32kb + ., :] Q^T.
  __device__ __forceinline__ static void scores(const uint16_t* kt, const FwdOffsets<D>& of,
                                                const bf16x8 (&qreg)[NKS], f32x16 (&sacc)[NKB]) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) sacc[kb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const bf16x8 a = lds_frag(kt + of.kfrag[ks] + 32 * kb * CPR * 8);
        sacc[kb] = mfma32(a, qreg[ks], sacc[kb]);
      }
    }
  }

  // Row max of one tile (when MASK, entries with key > lim are set to -inf;
  // lim is the last key this lane's row may see).
  template <bool MASK>
  __device__ __forceinline__ static float tile_max(f32x16 (&sacc)[NKB], int k0, int lim, int hh) {
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (MASK) {
          const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (key > lim) sacc[kb][r] = kNegInf;
        }
        mx = __builtin_fmaxf(mx, sacc[kb][r]);
      }
    }
    return __builtin_fmaxf(mx, wave_swap_halves(mx));
  }

  // P = exp2(S C - m) packed to bf16 for the PV product; fp32 row sum.
  template <bool MASK>
  __device__ __forceinline__ static void probs(const f32x16 (&sacc)[NKB], float C, float m, bf16x8 (&pb)[2 * NKB],
                                               float& l_part) {
    const float negm = -m;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        float p[8];
#pragma unroll
        for (int e8 = 0; e8 < 8; ++e8) {
          const int r = 8 * half + e8;
          float e = exp2_mode<EXPMODE>(__builtin_fmaf(sacc[kb][r], C, negm), r);
          if (MASK && sacc[kb][r] == kNegInf) e = 0.0f;
          p[e8] = e;
          l_part += e;
        }
        pb[2 * kb + half] = pack_probs(p);
      }
    }
  }

  // O^T += V^T P^T; the V^T operand comes from two LDS transpose loads of
  // four keys each: slots 0..3 -> keys 16t + 4h + s, 4..7 -> 16t + 8 + 4h + s-4.
  __device__ __forceinline__ static void pv(const uint16_t* vt, const FwdOffsets<D>& of,
                                            const bf16x8 (&pb)[2 * NKB], f32x16 (&oacc)[NDB]) {
    typedef short s16x8 __attribute__((ext_vector_type(8)));
#pragma unroll
    for (int t = 0; t < 2 * NKB; ++t) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(vt + of.vfrag[db][0] + 16 * t * CPR * 8));
        const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(vt + of.vfrag[db][1] + 16 * t * CPR * 8));
        const s16x8 v = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
        oacc[db] = mfma32(__builtin_bit_cast(bf16x8, v), pb[t], oacc[db]);
      }
    }
  }

  // One tile.  Region 1 (no branches): row max and the rescale decision,
  // the next tile's scores on the MFMA unit interleaved with this tile's
  // exponentials on the VALU.  Then the (rare) rescale of the output
  // accumulator, and region 2: P V with its transpose loads.  The next
  // tile's scores are computed even after the wave's last tile (from a
  // stale but finite buffer) so that region 1 has no branch.
  template <bool MASK>
  __device__ __forceinline__ static void step(const uint16_t* knext, const uint16_t* vcur, const FwdOffsets<D>& of,
                                              const bf16x8 (&qreg)[NKS], f32x16 (&scur)[NKB], f32x16 (&oacc)[NDB],
                                              float& m_run, float& l_part, int k0, int lim, int hh, float C,
                                              float tau) {
    f32x16 snext[NKB];
    bf16x8 pb[2 * NKB];
    const float mx = tile_max<MASK>(scur, k0, lim, hh);
    const float mxs = (mx == kNegInf) ? kNegInf : mx * C;
    const float m_new = __builtin_fmaxf(m_run, mxs);
    // conditional rescale: the wave moves its running max only when some
    // row's max grew by more than tau (always on the first tile)
    const bool grow = __any((m_new - m_run) > tau);
    const float alpha = (grow && m_new != kNegInf) ? exp2_native(m_run - m_new) : 1.0f;
    m_run = grow ? m_new : m_run;
    l_part *= alpha;
    scores(knext, of, qreg, snext);
    probs<MASK>(scur, C, m_run, pb, l_part);
#pragma unroll
    for (int i = 0; i < NKS * NKB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // six VALU
    }
    if (grow) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
    }
    pv(vcur, of, pb, oacc);
#pragma unroll
    for (int i = 0; i < 2 * NKB * NDB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);  // two LDS transpose reads
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);  // one MFMA
    }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) scur[kb] = snext[kb];
  }
};

// `causal` is a run-time argument: it only moves a few scalar bounds (tile
// order, tile counts, the last visible key), and one instantiation for both
// settings keeps the compiler from restructuring the non-causal loop into a
// version that spills registers.
template <int D, int EXPMODE>
__global__ __launch_bounds__(256, (D == 256) ? 1 : 2) void fwd_kernel(const uint16_t* __restrict__ Q,
                                                                      const uint16_t* __restrict__ K,
                                                                      const uint16_t* __restrict__ V,
                                                                      uint16_t* __restrict__ O,
                                                                      float* __restrict__ LSE, int BH, int S,
                                                                      float C, uint32_t qsign, float tau, int nqt,
                                                                      int causal) {
  using Cfg = FwdCfg<D>;
  using W = FwdWave<D, EXPMODE>;
  constexpr int BC = Cfg::BC, BR = Cfg::BR, NKB = Cfg::NKB, NKS = Cfg::NKS, NDB = Cfg::NDB;
  constexpr int TILE = Cfg::TILE_BYTES / 2;  // elements

  __shared__ __attribute__((aligned(1024))) uint16_t Kb[2][TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t Vb[2][TILE];

  // Heaviest causal query tiles first, all heads of one rank together; with
  // B*H a multiple of 8 every workgroup of one head lands on the same XCD.
  const int id = blockIdx.x;
  const int bh = id % BH;
  const int rank = id / BH;
  const int qt = causal ? (nqt - 1 - rank) : rank;
  const int q0 = qt * BR;
  const size_t base = (size_t)bh * (size_t)S * D;
  const uint16_t* Kh = K + base;
  const uint16_t* Vh = V + base;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int hh = lane >> 5;
  const int c32 = lane & 31;
  const int qw0 = q0 + wave * 32;  // first query of this wavefront
  const int qrow = qw0 + c32;      // this lane's query

  // Q^T operand, resident in registers: lane holds q[qrow][16ks + 8hh .. +7].
  bf16x8 qreg[NKS];
  {
    const u32x4* src = reinterpret_cast<const u32x4*>(Q + base + (size_t)min(qrow, S - 1) * D);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4 v = src[2 * ks + hh];
      v ^= qsign;
      qreg[ks] = as_bf16x8(v);
    }
  }

  const int kend = causal ? min(S, q0 + BR) : S;
  const int nkt = (kend + BC - 1) / BC;                                  // tiles of the workgroup
  const int nkt_w = causal ? min(nkt, (qw0 + 32 + BC - 1) / BC) : nkt;  // tiles this wave needs
  // Tiles [0, nfull) need no mask for this wave; the rest (diagonal or ragged) do.
  int nfull = causal ? (qw0 + 1) / BC : nkt_w;
  nfull = min(nfull, S / BC);

  // last key this lane's row may see (causal diagonal and/or end of sequence)
  const int lim = causal ? min(qrow, S - 1) : (S - 1);

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
  float m_run = kNegInf;  // running max, in units of log2 (scores times C)
  float l_part = 0.0f;    // this lane's partial row sum

  FwdOffsets<D> of;
  of.init(wave, lane);

  // prologue: K0, V0, K1 in flight; S^T(0) once K0 is in.
  dma_tile<D>(Kh, 0, S, Kb[0], wave, of.dma);
  dma_tile<D>(Vh, 0, S, Vb[0], wave, of.dma);
  if (nkt > 1) dma_tile<D>(Kh, BC, S, Kb[1], wave, of.dma);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  f32x16 scur[NKB];
  W::scores(Kb[0], of, qreg, scur);

  for (int kt = 0; kt < nkt; ++kt) {
    // loads for later tiles: K two ahead, V one ahead (buffers freed by the
    // barrier that ended the previous iteration)
    if (kt + 2 < nkt) dma_tile<D>(Kh, (kt + 2) * BC, S, Kb[kt & 1], wave, of.dma);
    if (kt + 1 < nkt) dma_tile<D>(Vh, (kt + 1) * BC, S, Vb[(kt + 1) & 1], wave, of.dma);
    __builtin_amdgcn_sched_barrier(0);  // keep the load issue out of the compute schedule

    if (kt < nkt_w) {
      if (kt < nfull)
        W::template step<false>(Kb[(kt + 1) & 1], Vb[kt & 1], of, qreg, scur, oacc, m_run, l_part, kt * BC, lim,
                                hh, C, tau);
      else
        W::template step<true>(Kb[(kt + 1) & 1], Vb[kt & 1], of, qreg, scur, oacc, m_run, l_part, kt * BC, lim,
                               hh, C, tau);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // ---- epilogue: O = acc / l, LSE = ln2 * (m + log2 l) ----------------------
  const float l_tot = l_part + wave_swap_halves(l_part);
  const float inv = 1.0f / l_tot;
  if (qrow < S) {
    uint16_t* orow = O + base + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * db + 8 * g + 4 * hh;
        *reinterpret_cast<u32x2*>(orow + d) =
            pack_bf16x4(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv, oacc[db][4 * g + 2] * inv,
                        oacc[db][4 * g + 3] * inv);
      }
    }
    if (hh == 0) LSE[(size_t)bh * S + qrow] = (m_run + __log2f(l_tot)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// exp2 diagnostic kernel: the same device exponentials, elementwise.
// ---------------------------------------------------------------------------
template <int MODE>
__global__ void exp2_eval_kernel(const float* __restrict__ x, float* __restrict__ y, long n) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) y[i] = (MODE == 1) ? exp2_poly(x[i]) : exp2_native(x[i]);
}

// ---------------------------------------------------------------------------
// host-side launchers
// ---------------------------------------------------------------------------
template <int D, int EXPMODE>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t st) {
  const int nqt = (a.S + FwdCfg<D>::BR - 1) / FwdCfg<D>::BR;
  const int BH = a.B * a.H;
  dim3 grid(nqt * BH), block(256);
  prof_begin(KID_FWD, st);
  hipLaunchKernelGGL((fwd_kernel<D, EXPMODE>), grid, block, 0, st,
                     (const uint16_t*)a.Q, (const uint16_t*)a.K, (const uint16_t*)a.V,
                     (uint16_t*)a.O, a.LSE, BH, a.S, a.C, a.qsign, a.tau, nqt, a.causal);
  prof_end(KID_FWD, st);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_fwd_e(const FwdArgs& a, hipStream_t st) {
  switch (a.exp_mode) {
    case 1: return launch_fwd_t<D, 1>(a, st);
    case 2: return launch_fwd_t<D, 2>(a, st);
    default: return launch_fwd_t<D, 0>(a, st);
  }
}

hipError_t launch_fwd(const FwdArgs& a, hipStream_t st) {
  switch (a.D) {
    case 64: return launch_fwd_e<64>(a, st);
    case 128: return launch_fwd_e<128>(a, st);
    case 256: return launch_fwd_e<256>(a, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_exp2_eval(const float* x, float* y, long n, int mode, hipStream_t st) {
  const long blocks = (n + 255) / 256;
  if (mode == 1)
    hipLaunchKernelGGL((exp2_eval_kernel<1>), dim3((unsigned)blocks), dim3(256), 0, st, x, y, n);
  else
    hipLaunchKernelGGL((exp2_eval_kernel<0>), dim3((unsigned)blocks), dim3(256), 0, st, x, y, n);
  return hipGetLastError();
}

}  // namespace attn97

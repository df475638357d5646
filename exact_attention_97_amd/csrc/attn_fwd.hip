// attn_fwd.hip - forward pass of exact attention on gfx950.
//
// One workgroup owns a tile of query rows of one (batch, head): eight
// wavefronts and 256 rows at D = 128 for long sequences (all eight share
// each K / V tile in LDS), four and 128 otherwise, at D = 64 and 256 and in
// the split-KV kernel.  Each
// wavefront owns 32 of those rows and walks the key/value sequence one tile
// of BC keys at a time:
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
// * K and V tiles go from HBM straight into LDS with LDS-direct buffer loads (16
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
// barrier per tile suffices; the eight-wavefront kernel puts two such
// steps in each LDS tile (one load issue and one barrier per 128 keys).
// One-query-row calls of the split-KV path
// (decoding) run splitkv_decode_kernel instead, which has no matrix tiles.
#include <stdlib.h>

#include <type_traits>

#include "attn_kernels.hpp"
#include "device_common.hpp"
#include "tile_layout.hpp"
#include "kv_stream.hpp"

namespace attn97 {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Default configurations per head dim (measured on MI355X).
template <int D>
struct FwdDefault;
template <>
struct FwdDefault<64> {
  using type = FwdCfg<64, 128, 4, 2>;
};
template <>
struct FwdDefault<128> {
  using type = FwdCfg<128, 64, 4, 2>;
};
template <>
struct FwdDefault<256> {
  using type = FwdCfg<256, 32, 4, 2>;
};

template <class Cfg, int EXPMODE>
struct FwdWave {
  static constexpr int D = Cfg::D, NKB = Cfg::NKB, NKS = Cfg::NKS, NDB = Cfg::NDB, BC = Cfg::BC, CPR = Cfg::CPR;

  // S^T of one tile: sacc[kb] = K[32kb + ., :] Q^T.
  __device__ __forceinline__ static void scores(const uint16_t* kt, const FwdOffsets<Cfg>& of,
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
  __device__ __forceinline__ static void pv(const uint16_t* vt, const FwdOffsets<Cfg>& of,
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

  // Schedule of the score MFMAs of the next tile interleaved with this
  // tile's softmax: the K fragment reads run four ahead of the MFMAs that use
  // them, and each MFMA is followed by NV VALU instructions.
  template <int NV>
  __device__ __forceinline__ static void region1_schedule() {
    constexpr int NS = NKS * NKB;  // score MFMAs of the next tile
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < NS - 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);
    }
  }

  // Where an unmasked tile's row max is taken: with eight wavefronts (the
  // D = 128 tile for long sequences) in the previous tile's region 2, under
  // its P V MFMAs (1.3 % faster at S = 8192); with four wavefronts in region
  // 1 (measured: neutral at D = 128, S = 4096, 1.5 % slower at D = 256, 7 %
  // at D = 64).
  static constexpr bool kMaxAhead = Cfg::NW == 8;

  // Region 1 of one tile (no branches): for a masked tile (diagonal or
  // ragged) the mask and the row max, for an unmasked one the row max (taken
  // in the previous tile's region 2, mx_pre, when kMaxAhead); the rescale
  // decision; then the
  // next tile's scores on the MFMA unit interleaved with this tile's
  // exponentials on the VALU.  Returns P (bf16) and the rescale decision for
  // region 2.  The next tile's scores are computed even after the wave's
  // last tile (from a stale buffer, never used) so that region 1 has no
  // branch.
  template <bool MASK>
  __device__ __forceinline__ static void region1(const uint16_t* knext, const FwdOffsets<Cfg>& of,
                                                 const bf16x8 (&qreg)[NKS], f32x16 (&scur)[NKB],
                                                 f32x16 (&snext)[NKB], float& m_run, float& l_part, int k0, int lim,
                                                 int hh, float C, float tau, float mx_pre, bf16x8 (&pb)[2 * NKB],
                                                 bool& grow, float& alpha) {
    const float mx = (MASK || !kMaxAhead) ? tile_max<MASK>(scur, k0, lim, hh) : mx_pre;
    const float mxs = (mx == kNegInf) ? kNegInf : mx * C;
    const float m_new = __builtin_fmaxf(m_run, mxs);
    // conditional rescale: the wave moves its running max only when some
    // row's max grew by more than tau (always on the first tile)
    grow = __any((m_new - m_run) > tau);
    alpha = (grow && m_new != kNegInf) ? exp2_native(m_run - m_new) : 1.0f;
    m_run = grow ? m_new : m_run;
    l_part *= alpha;
    // Region 1 runs at raised wave priority: of the two wavefronts sharing a
    // SIMD, the one issuing score MFMAs interleaved with softmax work is
    // preferred over one in its P V phase, which keeps the matrix unit fed.
    __builtin_amdgcn_s_setprio(1);
    scores(knext, of, qreg, snext);
    probs<MASK>(scur, C, m_run, pb, l_part);
    region1_schedule<6>();
    // keep the exponentials and the packed P above the (rare) rescale branch
#pragma unroll
    for (int t = 0; t < 2 * NKB; ++t) asm volatile("" ::"v"(__builtin_bit_cast(u32x4, pb[t])));
    asm volatile("" ::"v"(l_part));
    __builtin_amdgcn_s_setprio(0);
  }

  // P V with its transpose loads (the reads run eight ahead: two per MFMA
  // operand, so three MFMAs of look-ahead under the exact LDS wait counts),
  // and, with kMaxAhead, on the VALU meanwhile, the row max of the next
  // tile's scores (without the mask; a masked tile takes its own in region
  // 1).  Region 1 carries the whole softmax and this region none otherwise.
  __device__ __forceinline__ static void region2(const uint16_t* vcur, const FwdOffsets<Cfg>& of,
                                                 const bf16x8 (&pb)[2 * NKB], f32x16 (&oacc)[NDB],
                                                 f32x16 (&snext)[NKB], float& mx_next) {
    pv(vcur, of, pb, oacc);
    if constexpr (kMaxAhead) mx_next = tile_max<false>(snext, 0, 0, 0);
    constexpr int NP = 2 * NKB * NDB, PVA = 8;
    __builtin_amdgcn_sched_group_barrier(0x100, PVA, 1);
#pragma unroll
    for (int i = 0; i < NP - PVA / 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
      if constexpr (kMaxAhead) __builtin_amdgcn_sched_group_barrier(0x002, 2, 1);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, PVA / 2, 1);
    if constexpr (kMaxAhead) __builtin_amdgcn_sched_group_barrier(0x002, 8, 1);
  }

  // One whole tile: region 1, the (rare) rescale of the output accumulator,
  // region 2.  mx_pre: this tile's unmasked row max (from the previous
  // tile's region 2); mx_next: the next tile's, for the following step.
  template <bool MASK>
  __device__ __forceinline__ static void step(const uint16_t* knext, const uint16_t* vcur, const FwdOffsets<Cfg>& of,
                                              const bf16x8 (&qreg)[NKS], f32x16 (&scur)[NKB],
                                              f32x16 (&snext)[NKB], f32x16 (&oacc)[NDB], float& m_run,
                                              float& l_part, int k0, int lim, int hh, float C, float tau,
                                              float mx_pre, float& mx_next) {
    bf16x8 pb[2 * NKB];
    bool grow;
    float alpha;
    region1<MASK>(knext, of, qreg, scur, snext, m_run, l_part, k0, lim, hh, C, tau, mx_pre, pb, grow, alpha);
    if (grow) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
    }
    region2(vcur, of, pb, oacc, snext, mx_next);
  }
};

// Split-KV (SPLITKV): the keys are split into chunks of kchunk (a multiple
// of the tile) and workgroup (query tile, head, split) attends to one chunk,
// writing the chunk's normalised output (fp32) and log-sum-exp to
// workspace arrays that a merge kernel combines.  Queries and keys may then
// differ in length: S queries, Sk keys, and a causal query i sees keys up to
// i + Sk - S (the queries are the last S positions).
struct SplitKv {
  int Sk;        // number of keys (== S without SPLITKV)
  int kchunk;    // keys per split
  float* Opart;  // [nsplit, B*H, S, D] fp32
  float* Lpart;  // [nsplit, B*H, S] fp32, natural log; -inf for a row with no visible key
};

// `causal` is a run-time argument: it only moves a few scalar bounds (tile
// order, tile counts, the last visible key), and one instantiation for both
// settings keeps the compiler from restructuring the non-causal loop into a
// version that spills registers.
template <class Cfg, int EXPMODE, bool SPLITKV = false, int TW = 1>
__global__ __launch_bounds__(64 * Cfg::NW, (Cfg::D == 256 || Cfg::NW == 8) ? 1 : 2) void fwd_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int BH, int S, float C, uint32_t qsign, float tau, int nqt,
    int causal, SplitKv sk) {
  using W = FwdWave<Cfg, EXPMODE>;
  constexpr int D = Cfg::D, BC = Cfg::BC, BR = Cfg::BR, NKB = Cfg::NKB, NKS = Cfg::NKS, NDB = Cfg::NDB;
  constexpr int NBUF = Cfg::NBUF, DPW = Cfg::DMA_PER_WAVE;
  // LDS tiles of TW steps of BC keys (TW > 1: one load issue and one
  // barrier per TW steps)
  constexpr int TILE = Cfg::TILE_BYTES / 2 * TW;  // elements
  static_assert(TW == 1 || (NBUF == 2 && !SPLITKV), "multi-step tiles: two buffers, no split-KV");

  // One __shared__ array per buffer: with two buffers every buffer choice
  // below is a compile-time constant (the loop is unrolled by two), and the
  // compiler then sees that a tile load in flight cannot alias the buffer
  // being read (with one array indexed at run time it waits for all loads
  // before each read).
  __shared__ __attribute__((aligned(1024))) uint16_t Kb0[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t Kb1[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t Vb0[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t Vb1[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t Kb2[NBUF > 2 ? TILE : 8];
  __shared__ __attribute__((aligned(16))) uint16_t Vb2[NBUF > 2 ? TILE : 8];
  auto kbuf = [&](int i) -> uint16_t* { return i == 0 ? Kb0 : (i == 1 ? Kb1 : Kb2); };
  auto vbuf = [&](int i) -> uint16_t* { return i == 0 ? Vb0 : (i == 1 ? Vb1 : Vb2); };

  // Block order (xcd_head_order): one head's query tiles together on an XCD,
  // except for causal passes with fewer than 128 tiles per head and the
  // split-KV kernel, which take the grid-wide order (heaviest causal query
  // tiles first, all heads of one rank together; with B*H a multiple of 8
  // every workgroup of one head still lands on the same XCD).
  const int id = blockIdx.x;
  int bh, rank;
  if (SPLITKV) {
    bh = id % BH;
    rank = (id / BH) % nqt;
  } else {
    xcd_head_order(id, BH, nqt, !causal || nqt >= 128, bh, rank);
  }
  const int split = SPLITKV ? id / BH / nqt : 0;
  const int qt = causal ? (nqt - 1 - rank) : rank;
  const int q0 = qt * BR;
  const int Sk = SPLITKV ? sk.Sk : S;
  const int coff = Sk - S;                        // causal offset (0 when square)
  const int kb = SPLITKV ? split * sk.kchunk : 0;  // first key of this split
  const int ke = SPLITKV ? min(Sk, kb + sk.kchunk) : Sk;
  const size_t base = (size_t)bh * (size_t)S * D;
  const size_t kbase = (size_t)bh * (size_t)Sk * D;
  const uint16_t* Kh = K + kbase;
  const uint16_t* Vh = V + kbase;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  // the same index read from the first lane, for the LDS-DMA destinations
  // only (they must be uniform: with it they are scalar arithmetic, without
  // it every tile load pays a readfirstlane)
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
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
      // At D = 256 the kernel needs more than the 256 arch VGPRs; Q is read
      // only as an MFMA operand, which gfx950 takes from AGPRs, so it is
      // placed there once instead of being moved on every tile.
      if constexpr (D == 256) asm volatile("" : "+a"(v));
      qreg[ks] = as_bf16x8(v);
    }
  }

  // keys [kb, kend) are visible to some row of the workgroup; tile t covers
  // keys kb + t*BC ..
  const int kend = causal ? min(ke, q0 + BR + coff) : ke;
  const int nkt = kend > kb ? (kend - kb + BC - 1) / BC : 0;  // tiles of the workgroup
  const int wend = causal ? min(kend, qw0 + 32 + coff) : kend;
  // tiles this wave needs (none when all its rows are past the last query:
  // it still issues its share of the loads and takes part in the barriers)
  const int nkt_w = (wend > kb && qw0 < S) ? (wend - kb + BC - 1) / BC : 0;
  // Tiles [0, nfull) need no mask for this wave; the rest (diagonal or ragged) do.
  int nfull = causal ? (qw0 + coff + 1 - kb) / BC : nkt_w;
  nfull = max(0, min(nfull, (ke - kb) / BC));

  // last key this lane's row may see (causal diagonal, end of split / sequence)
  const int lim = causal ? min(qrow + coff, ke - 1) : (ke - 1);

  if constexpr (SPLITKV) {
    if (nkt == 0) {  // no key of this split is visible to the workgroup (uniform)
      if (qrow < S) {
        float* orow = sk.Opart + (((size_t)split * BH + bh) * S + qrow) * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * g + 4 * hh) = f32x4{};
        if (hh == 0) sk.Lpart[((size_t)split * BH + bh) * S + qrow] = kNegInf;
      }
      return;
    }
  }

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
  float m_run = kNegInf;  // running max, in units of log2 (scores times C)
  float l_part = 0.0f;    // this lane's partial row sum

  FwdOffsets<Cfg> of;
  of.init(wave, lane);

  if constexpr (TW > 1) {
    // Tiles of TW * BC keys.  V tile t holds keys TW BC t .. and K tile t
    // is offset by one step (keys TW BC t + BC ..): iteration t takes steps
    // TW t .. TW t + TW - 1, whose scores were computed one step earlier and
    // whose next-step scores come from K tile t, so each iteration reads one
    // K and one V tile and two buffers per kind suffice.  A tile is loaded
    // as TW tiles of BC keys (the swizzle repeats every 16 rows, so they
    // stack); a part starting at or past S is not loaded (its keys belong to
    // no step that is taken).
    constexpr int TK = TW * BC;
    const int ntt = (kend + TK - 1) / TK;
    auto load_parts = [&](const uint16_t* src, int k0, uint16_t* dst) {
#pragma unroll
      for (int h = 0; h < TW; ++h)
        if (k0 + h * BC < S) dma_tile<Cfg>(src, k0 + h * BC, S, dst + h * BC * D, wave_u, of.dma);
    };
    dma_tile<Cfg>(Kh, 0, S, Kb1, wave_u, of.dma);  // keys 0 .. BC-1: the first step's scores
    load_parts(Kh, BC, Kb0);
    load_parts(Vh, 0, Vb0);
    wait_vm_lds<0>();
    __syncthreads();
    f32x16 sa[NKB], sb[NKB];
    float ma = kNegInf, mb = kNegInf;
    W::scores(Kb1, of, qreg, sa);
    if constexpr (W::kMaxAhead) ma = W::template tile_max<false>(sa, 0, 0, 0);
    // iteration 0 reloads Kb1: every wave's reads of it must be complete first
    wait_vm_lds<63>();
    barrier_keep_loads();
    auto iteration = [&](int t, auto P) {
      constexpr int par = decltype(P)::value;
      const uint16_t* kc = par ? Kb1 : Kb0;
      const uint16_t* vc = par ? Vb1 : Vb0;
      if (t + 1 < ntt) {
        load_parts(Kh, TK * (t + 1) + BC, par ? Kb0 : Kb1);
        load_parts(Vh, TK * (t + 1), par ? Vb0 : Vb1);
      }
      __builtin_amdgcn_sched_barrier(0);  // keep the load issue out of the compute schedule
#pragma unroll
      for (int h = 0; h < TW; ++h) {
        const int kt = TW * t + h;
        f32x16(&scur)[NKB] = (h & 1) ? sb : sa;
        f32x16(&snext)[NKB] = (h & 1) ? sa : sb;
        float& mcur = (h & 1) ? mb : ma;
        float& mnext = (h & 1) ? ma : mb;
        if (kt < nkt_w) {
          if (kt < nfull)
            W::template step<false>(kc + h * BC * D, vc + h * BC * D, of, qreg, scur, snext, oacc, m_run, l_part,
                                    kt * BC, lim, hh, C, tau, mcur, mnext);
          else
            W::template step<true>(kc + h * BC * D, vc + h * BC * D, of, qreg, scur, snext, oacc, m_run, l_part,
                                   kt * BC, lim, hh, C, tau, mcur, mnext);
        }
      }
      wait_vm_lds<0>();
      barrier_keep_loads();
    };
    static_assert(TW % 2 == 0, "the score sets alternate per step");
    for (int t = 0; t < ntt; t += 2) {
      iteration(t, std::integral_constant<int, 0>{});
      if (t + 1 < ntt) iteration(t + 1, std::integral_constant<int, 1>{});
    }
  } else {
  // Load schedule: iteration j issues K(j + NBUF) and V(j + NBUF - 1) into
  // the buffers freed by the barrier of iteration j-1, and needs K(j + 1)
  // (scores of the next tile) and V(j).  The prologue issues what iterations
  // -NBUF..-1 would have.
  // ki, vi: the buffers of K(j + NBUF) and V(j + NBUF - 1)
  auto issue = [&](int j, int ki, int vi) {  // loads of "iteration" j; returns the number of ops issued
    int n = 0;
    if (j + NBUF < nkt) {
      dma_tile<Cfg>(Kh, kb + (j + NBUF) * BC, Sk, kbuf(ki), wave_u, of.dma);
      n += DPW;
    }
    if (j + NBUF - 1 >= 0 && j + NBUF - 1 < nkt) {
      dma_tile<Cfg>(Vh, kb + (j + NBUF - 1) * BC, Sk, vbuf(vi), wave_u, of.dma);
      n += DPW;
    }
    return n;
  };
  // Wait until only the loads of the latest issuing iteration are in flight
  // (three buffers) or none (two buffers).
  auto wait_loads = [&](int n_latest) {
    if (NBUF == 2 || n_latest == 0)
      wait_vm_lds<0>();
    else if (n_latest == DPW)
      wait_vm_lds<DPW>();
    else
      wait_vm_lds<2 * DPW>();
  };

  int n_last = 0;
  for (int j = -NBUF; j < 0; ++j) n_last = issue(j, (j + NBUF) % NBUF, (j + NBUF - 1 + NBUF) % NBUF);
  wait_loads(n_last);
  __syncthreads();

  // scores of the current and the next tile; the loop is unrolled by two so
  // that the two sets swap roles instead of being copied
  f32x16 sa[NKB], sb[NKB];
  float ma = kNegInf, mb = kNegInf;  // unmasked row maxima of the tiles in sa / sb
  W::scores(Kb0, of, qreg, sa);
  if constexpr (W::kMaxAhead) ma = W::template tile_max<false>(sa, 0, 0, 0);
  // iteration 0 reloads buffer 0 (with K(NBUF)): every wave's reads of K(0)
  // must be complete first
  wait_vm_lds<63>();
  barrier_keep_loads();

  // P = kt & 1 (the loop is unrolled by two); with two buffers all indices
  // follow from it at compile time
  auto iteration = [&](int kt, auto P, f32x16(&scur)[NKB], f32x16(&snext)[NKB], float& mcur, float& mnext) {
    constexpr int par = decltype(P)::value;
    const int kn = NBUF == 2 ? 1 - par : (kt + 1) % NBUF;  // K(kt + 1)
    const int vc = NBUF == 2 ? par : kt % NBUF;            // V(kt)
    const int ki = NBUF == 2 ? par : kt % NBUF;            // K(kt + NBUF)
    const int vi = NBUF == 2 ? 1 - par : (kt + NBUF - 1) % NBUF;  // V(kt + NBUF - 1)
    n_last = issue(kt, ki, vi);
    __builtin_amdgcn_sched_barrier(0);  // keep the load issue out of the compute schedule
    if (kt < nkt_w) {
      if (kt < nfull)
        W::template step<false>(kbuf(kn), vbuf(vc), of, qreg, scur, snext, oacc, m_run, l_part, kb + kt * BC, lim,
                                hh, C, tau, mcur, mnext);
      else
        W::template step<true>(kbuf(kn), vbuf(vc), of, qreg, scur, snext, oacc, m_run, l_part, kb + kt * BC, lim,
                               hh, C, tau, mcur, mnext);
    }
    wait_loads(n_last);
    barrier_keep_loads();
  };
  for (int kt = 0; kt < nkt; kt += 2) {
    iteration(kt, std::integral_constant<int, 0>{}, sa, sb, ma, mb);
    if (kt + 1 < nkt) iteration(kt + 1, std::integral_constant<int, 1>{}, sb, sa, mb, ma);
  }
  }  // TW == 1

// ---- epilogue: O = acc / l, LSE = ln2 * (m + log2 l) ----------------------
  const float l_tot = l_part + wave_swap_halves(l_part);
  if constexpr (SPLITKV) {  // a row may see no key of this split: O = 0, LSE = -inf
    const bool any = l_tot > 0.0f;
    const float inv = any ? 1.0f / l_tot : 0.0f;
    if (qrow < S) {
      float* orow = sk.Opart + (((size_t)split * BH + bh) * S + qrow) * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * g + 4 * hh) =
              f32x4{oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv, oacc[db][4 * g + 2] * inv,
                    oacc[db][4 * g + 3] * inv};
      if (hh == 0) sk.Lpart[((size_t)split * BH + bh) * S + qrow] = any ? (m_run + __log2f(l_tot)) * kLn2 : kNegInf;
    }
    return;
  }
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
// Split-KV decoding: one query row per head (Sq = 1), where the MFMA tiles of
// fwd_kernel would compute 31 padding rows of every 32 and the work is
// reading K and V.  Workgroup (split, head), four wavefronts; lane
// (g, c) holds the 16-byte column chunk c (elements 8 c .. 8 c + 7) of key
// slot g, so D / 8 lanes cover one key row and a wavefront reads
// 64 * 8 / D consecutive keys per step, eight steps of K and V loads in flight
// before any arithmetic.  Scores are fp32 dot products reduced across the
// row's lanes; the running max and sum are per wavefront (the accumulator is
// rescaled once per eight steps, exactly, with no threshold); the four
// wavefronts combine through LDS into the split's normalised output and
// log-sum-exp, the format the merge kernel reads.  With one query row and
// the queries read as the last positions, every key is visible, causal or
// not.  Exponentials are native.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void splitkv_decode_kernel(const uint16_t* __restrict__ Q,
                                                             const uint16_t* __restrict__ K,
                                                             const uint16_t* __restrict__ V, int BH, int Sk,
                                                             int kchunk, float C, uint32_t qsign,
                                                             float* __restrict__ Opart, float* __restrict__ Lpart) {
  constexpr int LPK = D / 8;     // lanes per key row
  constexpr int KPW = 64 / LPK;  // keys per wavefront per step
  constexpr int U = 8;           // steps loaded before computing
  __shared__ float wm[4], wl[4];
  __shared__ float wacc[4][D];
  const int id = blockIdx.x;
  const int bh = id % BH, split = id / BH;
  const int kb = split * kchunk, ke = min(Sk, kb + kchunk);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane / LPK, c = lane % LPK;
  const uint16_t* Kh = K + (size_t)bh * Sk * D + 8 * c;
  const uint16_t* Vh = V + (size_t)bh * Sk * D + 8 * c;

  float q[8];
  {
    u32x4 w = *reinterpret_cast<const u32x4*>(Q + (size_t)bh * D + 8 * c);
    w ^= qsign;  // a negative scale flips the sign of q
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      q[2 * e] = __builtin_bit_cast(float, w[e] << 16);
      q[2 * e + 1] = __builtin_bit_cast(float, w[e] & 0xFFFF0000u);
    }
  }
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
  float m_run = kNegInf;  // log2 units
  float l = 0.0f;         // sum of this lane's key slot's probabilities

  const int nstep = (ke - kb + 4 * KPW - 1) / (4 * KPW);  // steps of the workgroup
  for (int it0 = 0; it0 < nstep; it0 += U) {
    u32x4 kw[U], vw[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int key = kb + ((it0 + u) * 4 + wave) * KPW + g;
      ok[u] = key < ke;  // covers steps past the end too
      kw[u] = ok[u] ? *reinterpret_cast<const u32x4*>(Kh + (size_t)key * D) : u32x4{0, 0, 0, 0};
      vw[u] = ok[u] ? *reinterpret_cast<const u32x4*>(Vh + (size_t)key * D) : u32x4{0, 0, 0, 0};
    }
    float sc[U];
    float mx = kNegInf;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float dot = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dot = __builtin_fmaf(q[2 * e], __builtin_bit_cast(float, kw[u][e] << 16), dot);
        dot = __builtin_fmaf(q[2 * e + 1], __builtin_bit_cast(float, kw[u][e] & 0xFFFF0000u), dot);
      }
#pragma unroll
      for (int o = 1; o < LPK; o <<= 1) dot += __shfl_xor(dot, o);
      sc[u] = ok[u] ? dot * C : kNegInf;
      mx = __builtin_fmaxf(mx, sc[u]);
    }
#pragma unroll
    for (int o = LPK; o < 64; o <<= 1) mx = __builtin_fmaxf(mx, __shfl_xor(mx, o));
    const float m_new = __builtin_fmaxf(m_run, mx);
    if (m_new == kNegInf) continue;  // no key of this wavefront in these steps (wave-uniform)
    const float alpha = exp2_native(m_run - m_new);  // 0 on the first keys (m_run = -inf)
    l *= alpha;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] *= alpha;
    m_run = m_new;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float p = ok[u] ? exp2_native(sc[u] - m_run) : 0.0f;
      l += p;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] = __builtin_fmaf(p, __builtin_bit_cast(float, vw[u][e] << 16), acc[2 * e]);
        acc[2 * e + 1] = __builtin_fmaf(p, __builtin_bit_cast(float, vw[u][e] & 0xFFFF0000u), acc[2 * e + 1]);
      }
    }
  }
  // sum over the key slots of the wavefront (lanes with equal c)
#pragma unroll
  for (int o = LPK; o < 64; o <<= 1) {
    l += __shfl_xor(l, o);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] += __shfl_xor(acc[j], o);
  }
  if (lane < LPK) {
#pragma unroll
    for (int j = 0; j < 8; ++j) wacc[wave][8 * lane + j] = acc[j];
  }
  if (lane == 0) {
    wm[wave] = m_run;
    wl[wave] = l;
  }
  __syncthreads();
  if (tid < D) {
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = __builtin_fmaxf(M, wm[w]);
    float L = 0.0f, o = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = (wm[w] == kNegInf) ? 0.0f : exp2_native(wm[w] - M);
      L += f * wl[w];
      o += f * wacc[w][tid];
    }
    // the split holds at least one key (kb < Sk), so M is finite and L > 0
    Opart[((size_t)split * BH + bh) * D + tid] = o / L;
    if (tid == 0) Lpart[(size_t)split * BH + bh] = (M + __log2f(L)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// Split-KV merge: per row, LSE = ln sum_c exp(LSE_c) and
// O = sum_c exp(LSE_c - LSE) O_c, rounded to bf16 (the decomposition of the
// softmax over disjoint key sets that also makes LSE an output of the
// forward pass).  D/4 threads per row, four columns each; HBM-bound.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void splitkv_merge_kernel(const float* __restrict__ Opart,
                                                            const float* __restrict__ Lpart, uint16_t* __restrict__ O,
                                                            float* __restrict__ LSE, long rows, int nsplit) {
  constexpr int TPR = D / 4;
  const long row = ((long)blockIdx.x * 256 + threadIdx.x) / TPR;
  const int c = threadIdx.x % TPR;
  if (row >= rows) return;
  float m = kNegInf;
  for (int sp = 0; sp < nsplit; ++sp) m = __builtin_fmaxf(m, Lpart[(size_t)sp * rows + row]);
  f32x4 acc = f32x4{};
  float wsum = 0.0f;
  for (int sp = 0; sp < nsplit; ++sp) {
    const float l = Lpart[(size_t)sp * rows + row];
    const float w = (l == kNegInf) ? 0.0f : exp2_native((l - m) * kLog2e);  // the largest term has w = 1
    const f32x4 o = *reinterpret_cast<const f32x4*>(Opart + ((size_t)sp * rows + row) * D + 4 * c);
    acc += w * o;
    wsum += w;
  }
  const float inv = 1.0f / wsum;
  *reinterpret_cast<u32x2*>(O + (size_t)row * D + 4 * c) =
      pack_bf16x4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
  if (c == 0) LSE[row] = m + __log2f(wsum) * kLn2;
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
template <class Cfg, int EXPMODE, int TW = 1>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t st) {
  const int nqt = (a.S + Cfg::BR - 1) / Cfg::BR;
  const int BH = a.B * a.H;
  dim3 grid(nqt * BH), block(64 * Cfg::NW);
  prof_begin(KID_FWD, st);
  hipLaunchKernelGGL((fwd_kernel<Cfg, EXPMODE, false, TW>), grid, block, 0, st, (const uint16_t*)a.Q, (const uint16_t*)a.K,
                     (const uint16_t*)a.V, (uint16_t*)a.O, a.LSE, BH, a.S, a.C, a.qsign, a.tau, nqt, a.causal,
                     SplitKv{a.S, 0, nullptr, nullptr});
  prof_end(KID_FWD, st);
  return hipGetLastError();
}

// a.exp_mode is the kernel exp2 mode (kExpNative, kExpPoly or exp_mix(q)).
template <class Cfg, int TW = 1>
static hipError_t launch_fwd_e(const FwdArgs& a, hipStream_t st) {
  switch (a.exp_mode) {
    case kExpPoly: return launch_fwd_t<Cfg, kExpPoly, TW>(a, st);
    case exp_mix(1): return launch_fwd_t<Cfg, exp_mix(1), TW>(a, st);
    case exp_mix(2): return launch_fwd_t<Cfg, exp_mix(2), TW>(a, st);
    case exp_mix(3): return launch_fwd_t<Cfg, exp_mix(3), TW>(a, st);
    default: return launch_fwd_t<Cfg, kExpNative, TW>(a, st);
  }
}

// The D = 128 tile (measured on MI355X, B=2, H=16, outlier inputs, S from
// 2048 to 8192 in steps of 1024).  The cooperative big tile, eight
// wavefronts (256 queries) sharing each K / V tile in LDS with two 64-key
// steps per LDS tile, is 3-3.5 % faster than four wavefronts (128 queries,
// two workgroups per CU) when its workgroups fill whole rounds of the CUs
// (S = 4096, 6144, 8192 at B*H = 32) and 1-8 % slower when the last round
// is partial (S = 3072, 5120, 7168), where the smaller workgroups balance
// better; at S = 2048 four wavefronts are 8 % faster causal.  So: eight
// wavefronts from S = 4096 on when the 256-query workgroups are a multiple
// of the CU count, else four.  Variant 1 (attn_set_variant("fwd", 1) or
// ATTN97_FWD_VARIANT=1) takes the eight-wavefront tile at every length, so
// that its ragged and short cases can be tested.  Split-KV keeps four,
// which suits few query rows.
static int fwd_variant() { return kernel_variant(VAR_FWD); }

// Compute units of the current device (cached per device).
static int device_cus() {
  static int cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    cus[dev] = (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0) ? n : 256;
  }
  return cus[dev];
}

static bool fwd_big_tile(const FwdArgs& a) {
  if (fwd_variant() == 1) return true;
  if (fwd_variant() == 2) return false;
  const long wgs = (long)((a.S + 255) / 256) * a.B * a.H;
  return a.S >= 4096 && wgs % device_cus() == 0;
}

hipError_t launch_fwd(const FwdArgs& a, hipStream_t st) {
  switch (a.D) {
    case 64: return launch_fwd_e<FwdDefault<64>::type>(a, st);
    case 128:
      if (fwd_big_tile(a)) return launch_fwd_e<FwdCfg<128, 64, 8, 2>, 2>(a, st);
      return launch_fwd_e<FwdDefault<128>::type>(a, st);
    case 256: return launch_fwd_e<FwdDefault<256>::type>(a, st);
    default: return hipErrorInvalidValue;
  }
}

int fwd_tile_keys(int D) {
  switch (D) {
    case 64: return FwdDefault<64>::type::BC;
    case 128: return FwdDefault<128>::type::BC;
    case 256: return FwdDefault<256>::type::BC;
    default: return 0;
  }
}

int fwd_tile_queries(int D) {
  switch (D) {
    case 64: return FwdDefault<64>::type::BR;
    case 128: return FwdDefault<128>::type::BR;
    case 256: return FwdDefault<256>::type::BR;
    default: return 0;
  }
}

template <class Cfg, int EXPMODE>
static hipError_t launch_splitkv_t(const FwdArgs& a, const SplitKvLaunch& p, hipStream_t st) {
  const int nqt = (a.S + Cfg::BR - 1) / Cfg::BR;
  const int BH = a.B * a.H;
  prof_begin(KID_FWD_SPLITKV, st);
  hipLaunchKernelGGL((fwd_kernel<Cfg, EXPMODE, true>), dim3(nqt * BH * p.nsplit), dim3(64 * Cfg::NW), 0, st,
                     (const uint16_t*)a.Q, (const uint16_t*)a.K, (const uint16_t*)a.V, (uint16_t*)a.O, a.LSE, BH,
                     a.S, a.C, a.qsign, a.tau, nqt, a.causal, SplitKv{p.Sk, p.kchunk, p.Opart, p.Lpart});
  prof_end(KID_FWD_SPLITKV, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long rows = (long)BH * a.S;
  const long threads = rows * (Cfg::D / 4);
  prof_begin(KID_SPLITKV_MERGE, st);
  hipLaunchKernelGGL((splitkv_merge_kernel<Cfg::D>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st,
                     (const float*)p.Opart, (const float*)p.Lpart, (uint16_t*)a.O, a.LSE, rows, p.nsplit);
  prof_end(KID_SPLITKV_MERGE, st);
  return hipGetLastError();
}

template <class Cfg>
static hipError_t launch_splitkv_e(const FwdArgs& a, const SplitKvLaunch& p, hipStream_t st) {
  switch (a.exp_mode) {
    case kExpPoly: return launch_splitkv_t<Cfg, kExpPoly>(a, p, st);
    case exp_mix(1): return launch_splitkv_t<Cfg, exp_mix(1)>(a, p, st);
    case exp_mix(2): return launch_splitkv_t<Cfg, exp_mix(2)>(a, p, st);
    case exp_mix(3): return launch_splitkv_t<Cfg, exp_mix(3)>(a, p, st);
    default: return launch_splitkv_t<Cfg, kExpNative>(a, p, st);
  }
}

template <int D>
static hipError_t launch_decode_t(const FwdArgs& a, const SplitKvLaunch& p, hipStream_t st) {
  const int BH = a.B * a.H;
  prof_begin(KID_FWD_SPLITKV, st);
  hipLaunchKernelGGL((splitkv_decode_kernel<D>), dim3(BH * p.nsplit), dim3(256), 0, st, (const uint16_t*)a.Q,
                     (const uint16_t*)a.K, (const uint16_t*)a.V, BH, p.Sk, p.kchunk, a.C, a.qsign, p.Opart, p.Lpart);
  prof_end(KID_FWD_SPLITKV, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long rows = (long)BH;
  const long threads = rows * (D / 4);
  prof_begin(KID_SPLITKV_MERGE, st);
  hipLaunchKernelGGL((splitkv_merge_kernel<D>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st,
                     (const float*)p.Opart, (const float*)p.Lpart, (uint16_t*)a.O, a.LSE, rows, p.nsplit);
  prof_end(KID_SPLITKV_MERGE, st);
  return hipGetLastError();
}

hipError_t launch_fwd_splitkv(const FwdArgs& a, const SplitKvLaunch& p, hipStream_t st) {
  if (a.S == 1) {  // decoding: one query row per head
    switch (a.D) {
      case 64: return launch_decode_t<64>(a, p, st);
      case 128: return launch_decode_t<128>(a, p, st);
      case 256: return launch_decode_t<256>(a, p, st);
      default: return hipErrorInvalidValue;
    }
  }
  switch (a.D) {
    case 64: return launch_splitkv_e<FwdDefault<64>::type>(a, p, st);
    case 128: return launch_splitkv_e<FwdDefault<128>::type>(a, p, st);
    case 256: return launch_splitkv_e<FwdDefault<256>::type>(a, p, st);
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

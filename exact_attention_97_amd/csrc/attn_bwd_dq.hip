// attn_bwd_dq.hip - dQ of the split backward pass (no atomics).
//
// The atomic backward pass adds every key tile's contribution to dQ with
// fp32 atomics; the pages name those atomic additions as an overhead of the
// backward pass at long sequence lengths (page "FlashAttention-3 и
// FlashAttention-4", section "Режим 2-CTA MMA"; abstract of
// "FlashAttention-4: Algorithm and Kernel Pipelining Co-Design for
// Asymmetric Hardware Scaling").  The split backward pass instead forms dK
// and dV in one kernel (per key tile) and dQ here, per query tile, walking
// the key sequence like the forward pass and recomputing what dQ needs:
//
//   Delta = rowsum(dO O), -LSE log2e   (per query row, also written out for
//                                       the dK/dV kernel, launched after this one)
//   S^T  = K Q^T           dP^T = V dO^T           (bf16 MFMA)
//   P    = exp2(S c - LSE log2e)                   (per lane: one query)
//   dS   = P (dP - Delta)
//   dQ^T += K^T dS^T      (K^T by LDS transpose loads, dS^T from registers)
//
// then dQ = scale * acc in bf16.  No atomics; the result is deterministic.
// Three products per tile instead of the atomic kernel's one for dQ.
#include <stdlib.h>

#include <type_traits>

#include "attn_kernels.hpp"
#include "device_common.hpp"
#include "kv_stream.hpp"
#include "tile_layout.hpp"

namespace attn97 {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

// Two 32-key blocks per tile, software-pipelined like the dK/dV tile:
//   A: S^T, dP^T of block 0
//   B: S^T, dP^T of block 1   | softmax of block 0
//   C: dQ^T with block 0      | softmax of block 1
//   D: dQ^T with block 1
// Source-level chunks separated by scheduling barriers fix the interleave;
// operand reads are issued one chunk ahead.
template <class Cfg>
struct DqWavePipe {
  static constexpr int D = Cfg::D, NKS = Cfg::NKS, NDB = Cfg::NDB, CPR = Cfg::CPR;
  static_assert(Cfg::NKB == 2, "two 32-key blocks per tile");
  // softmax elements (16 per block) per chunk of phase B (one reduction step
  // of the S and dP products)
  static constexpr int EB = 16 / NKS;
  static_assert(EB * NKS == 16 && 8 % NDB == 0, "elements spread evenly over the chunks");

  template <bool MASK>
  __device__ __forceinline__ static void elem(const f32x16& sacc, const f32x16& dpacc, int r, float C, float nlse2,
                                              float dlt, int key, int lim, float& ds) {
    float p = exp2_native(__builtin_fmaf(sacc[r], C, nlse2));
    if (MASK) p = (key > lim) ? 0.0f : p;
    ds = p * (dpacc[r] - dlt);
  }

  template <bool MASK>
  __device__ __forceinline__ static void step(const uint16_t* kt, const uint16_t* vt, const FwdOffsets<Cfg>& of,
                                              const bf16x8 (&qreg)[NKS], const bf16x8 (&doreg)[NKS],
                                              f32x16 (&dqacc)[NDB], float C, float nlse2, float dlt, int k0,
                                              int lim, int hh) {
    tile_marker<MASK>();
    auto kfrag = [&](int kb, int ks) { return lds_frag(kt + of.kfrag[ks] + 32 * kb * CPR * 8); };
    auto vfrag = [&](int kb, int ks) { return lds_frag(vt + of.kfrag[ks] + 32 * kb * CPR * 8); };
    auto ktr = [&](int t, int db) {  // K^T operand of the 16 keys of step t
      const int o = 16 * t * CPR * 8;
      const s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(kt + of.vfrag[db][0] + o));
      const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(kt + of.vfrag[db][1] + o));
      const s16x8 v = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
      return __builtin_bit_cast(bf16x8, v);
    };
    // key of accumulator register r in block kb
    auto keyof = [&](int kb, int r) { return k0 + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3); };

    f32x16 s0 = f32x16{}, dp0 = f32x16{}, s1 = f32x16{}, dp1 = f32x16{};
    float ds[16];
    bf16x8 dsb0[2], dsb1[2];

    {  // A
      bf16x8 ka[NKS], va[NKS];
      ka[0] = kfrag(0, 0); va[0] = vfrag(0, 0);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        if (ks + 1 < NKS) { ka[ks + 1] = kfrag(0, ks + 1); va[ks + 1] = vfrag(0, ks + 1); }
        s0 = mfma32(ka[ks], qreg[ks], s0);
        dp0 = mfma32(va[ks], doreg[ks], dp0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    {  // B
      bf16x8 ka[NKS], va[NKS];
      ka[0] = kfrag(1, 0); va[0] = vfrag(1, 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {  // EB of block 0's 16 elements per reduction step
        if (ks + 1 < NKS) { ka[ks + 1] = kfrag(1, ks + 1); va[ks + 1] = vfrag(1, ks + 1); }
        s1 = mfma32(ka[ks], qreg[ks], s1);
#pragma unroll
        for (int e = 0; e < (EB + 1) / 2; ++e) {
          const int r = EB * ks + e;
          elem<MASK>(s0, dp0, r, C, nlse2, dlt, keyof(0, r), lim, ds[r]);
        }
        dp1 = mfma32(va[ks], doreg[ks], dp1);
#pragma unroll
        for (int e = (EB + 1) / 2; e < EB; ++e) {
          const int r = EB * ks + e;
          elem<MASK>(s0, dp0, r, C, nlse2, dlt, keyof(0, r), lim, ds[r]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      dsb0[0] = pack_probs(*reinterpret_cast<float(*)[8]>(&ds[0]));
      dsb0[1] = pack_probs(*reinterpret_cast<float(*)[8]>(&ds[8]));
    }
    // Block 1's elements: at D = 64 and 256, 0 .. 7 (the first k-step of its
    // dQ product) over phase C's 2 NDB MFMAs and 8 .. 15 over the first NDB
    // MFMAs of phase D, which need only elements 0 .. 7 (same-process A/B:
    // dQ 3 % faster at D = 256, 0.7 % at D = 64); at D = 128 all sixteen
    // over phase C (the split measured 0.4-0.7 % slower there)
    constexpr int NC = D == 128 ? 16 : 8;  // block 1 elements in phase C
    {  // C
      bf16x8 ta[2 * NDB];
      ta[0] = ktr(0, 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 2 * NDB; ++i) {  // i = NDB t + db
        const int t = i / NDB, db = i % NDB;
        if (i + 1 < 2 * NDB) ta[i + 1] = ktr((i + 1) / NDB, (i + 1) % NDB);
        dqacc[db] = mfma32(ta[i], t == 0 ? dsb0[0] : dsb0[1], dqacc[db]);
#pragma unroll
        for (int r = NC * i / (2 * NDB); r < NC * (i + 1) / (2 * NDB); ++r)
          elem<MASK>(s1, dp1, r, C, nlse2, dlt, keyof(1, r), lim, ds[r]);
        __builtin_amdgcn_sched_barrier(0);
      }
      dsb1[0] = pack_probs(*reinterpret_cast<float(*)[8]>(&ds[0]));
      if constexpr (NC == 16) dsb1[1] = pack_probs(*reinterpret_cast<float(*)[8]>(&ds[8]));
    }
    {  // D
      bf16x8 ta[2 * NDB];
      ta[0] = ktr(2, 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 2 * NDB; ++i) {
        const int t = i / NDB, db = i % NDB;
        if (i + 1 < 2 * NDB) ta[i + 1] = ktr(2 + (i + 1) / NDB, (i + 1) % NDB);
        dqacc[db] = mfma32(ta[i], t == 0 ? dsb1[0] : dsb1[1], dqacc[db]);
        if (NC == 8 && i < NDB) {
#pragma unroll
          for (int r = 8 + 8 * i / NDB; r < 8 + 8 * (i + 1) / NDB; ++r)
            elem<MASK>(s1, dp1, r, C, nlse2, dlt, keyof(1, r), lim, ds[r]);
          if (i == NDB - 1) dsb1[1] = pack_probs(*reinterpret_cast<float(*)[8]>(&ds[8]));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
};

template <class Cfg, int OCC, int TW = 1>
__global__ __launch_bounds__(64 * Cfg::NW, OCC) void bwd_dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const uint16_t* __restrict__ O, const float* __restrict__ LSE,
    float* __restrict__ nlse2v, float* __restrict__ delta, uint16_t* __restrict__ dQ, int BH, int S, float scale,
    float C, int nqt, int causal) {
  using W = DqWavePipe<Cfg>;
  constexpr int D = Cfg::D, BC = Cfg::BC, BR = Cfg::BR, NKS = Cfg::NKS, NDB = Cfg::NDB;
  // LDS tiles of TW steps of BC keys (one load issue and one barrier per TW steps)
  using CfgT = FwdCfg<D, BC * TW, Cfg::NW, 2>;
  constexpr int TILE = CfgT::TILE_BYTES / 2;

  // one __shared__ array per buffer; the loop below is unrolled by two, so
  // every buffer a tile reads or loads into is a compile-time constant (LDS
  // addresses become instruction immediates, and the compiler can see that
  // the next tile's loads do not alias this tile's reads)
  __shared__ __attribute__((aligned(1024))) uint16_t Kb0[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t Kb1[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t Vb0[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t Vb1[TILE];

  // block order (xcd_head_order): one head's query tiles together on an XCD,
  // except for causal passes with fewer than 128 tiles per head, which run
  // the heaviest query tiles of all heads first
  int bh, rank;
  xcd_head_order(blockIdx.x, BH, nqt, !causal || nqt >= 128, bh, rank);
  const int qt = causal ? (nqt - 1 - rank) : rank;
  const int q0 = qt * BR;
  const size_t base = (size_t)bh * (size_t)S * D;
  const uint16_t* Kh = K + base;
  const uint16_t* Vh = V + base;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  // the same index read from the first lane, for the LDS-DMA destinations
  // only (they must be uniform: with it they are scalar arithmetic, without
  // it every tile load pays a readfirstlane)
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int lane = tid & 63;
  const int hh = lane >> 5;
  const int c32 = lane & 31;
  const int qw0 = q0 + wave * 32;
  const int qrow = qw0 + c32;
  const int qc = min(qrow, S - 1);

  // Q^T and dO^T operands in registers: lane holds row qrow, d = 16 ks + 8 h ..
  bf16x8 qreg[NKS], doreg[NKS];
  // Delta of this lane's row, sum_d dO_d O_d: each lane of the pair (l, l+32)
  // takes the half of the row it holds as the dO operand
  float dlt = 0.0f;
  {
    const u32x4* qs = reinterpret_cast<const u32x4*>(Q + base + (size_t)qc * D);
    const u32x4* ds = reinterpret_cast<const u32x4*>(dO + base + (size_t)qc * D);
    const u32x4* os = reinterpret_cast<const u32x4*>(O + base + (size_t)qc * D);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const u32x4 g = ds[2 * ks + hh], o = os[2 * ks + hh];
      qreg[ks] = as_bf16x8(qs[2 * ks + hh]);
      doreg[ks] = as_bf16x8(g);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        dlt = __builtin_fmaf(__uint_as_float(o[m] << 16), __uint_as_float(g[m] << 16), dlt);
        dlt = __builtin_fmaf(__uint_as_float(o[m] & 0xffff0000u), __uint_as_float(g[m] & 0xffff0000u), dlt);
      }
    }
    // At D = 256 the kernel needs more than the 256 arch VGPRs.  Q and dO are
    // read only as MFMA operands, which gfx950 takes from AGPRs, so their 128
    // registers are placed there once; otherwise the allocator moves values
    // between VGPRs and AGPRs on every tile.
    if constexpr (D == 256) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        u32x4 a = __builtin_bit_cast(u32x4, qreg[ks]), b = __builtin_bit_cast(u32x4, doreg[ks]);
        asm volatile("" : "+a"(a), "+a"(b));
        qreg[ks] = __builtin_bit_cast(bf16x8, a);
        doreg[ks] = __builtin_bit_cast(bf16x8, b);
      }
    }
  }
  dlt += wave_swap_halves(dlt);
  const float nlse2 = -LSE[(size_t)bh * S + qc] * kLog2e;  // -LSE log2(e)
  // the dK/dV kernel, launched after this one, reads both per row
  if (qrow < S && hh == 0) {
    delta[(size_t)bh * S + qrow] = dlt;
    nlse2v[(size_t)bh * S + qrow] = nlse2;
  }

  const int kend = causal ? min(S, q0 + BR) : S;
  const int nkt = (kend + BC - 1) / BC;
  const int nkt_w = causal ? min(nkt, (qw0 + 32 + BC - 1) / BC) : nkt;
  int nfull = causal ? (qw0 + 1) / BC : nkt_w;
  nfull = min(nfull, S / BC);
  const int lim = causal ? min(qrow, S - 1) : (S - 1);

  FwdOffsets<Cfg> of;
  of.init(wave, lane);
  const int ntt = (kend + BC * TW - 1) / (BC * TW);  // LDS tiles

  f32x16 dqacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dqacc[db] = f32x16{};

  // a TW-step tile is loaded as TW tiles of BC keys (the swizzle repeats
  // every 16 rows, so they stack); a part starting at or past S is not
  // loaded (its step is never taken, and dma_tile needs k0 < S)
  auto load_tile = [&](int k0, uint16_t* kd, uint16_t* vd) {
#pragma unroll
    for (int h = 0; h < TW; ++h) {
      if (h == 0 || k0 + h * BC < S) {
        dma_tile<Cfg>(Kh, k0 + h * BC, S, kd + h * BC * D, wave_u, of.dma);
        dma_tile<Cfg>(Vh, k0 + h * BC, S, vd + h * BC * D, wave_u, of.dma);
      }
    }
  };
  load_tile(0, Kb0, Vb0);
  wait_vm_lds<0>();
  barrier_keep_loads();

  // P = kt & 1: tile kt sits in buffer P, tile kt + 1 goes to the other one
  // (last read in the previous iteration)
  auto iteration = [&](int tt, auto P) {
    constexpr int par = decltype(P)::value;
    const uint16_t* kc = par ? Kb1 : Kb0;
    const uint16_t* vc = par ? Vb1 : Vb0;
    if (tt + 1 < ntt) load_tile((tt + 1) * BC * TW, par ? Kb0 : Kb1, par ? Vb0 : Vb1);
    __builtin_amdgcn_sched_barrier(0);
    // The offsets pass through an empty asm at each step: the compiler then
    // cannot precompute both buffers' addresses and hold them over the loop
    // (it adds the constant buffer base as the instruction's immediate).
    auto fresh_offsets = [&]() {
#pragma unroll
      for (int ks = 0; ks < Cfg::NKS; ++ks) asm volatile("" : "+v"(of.kfrag[ks]));
#pragma unroll
      for (int db = 0; db < Cfg::NDB; ++db) asm volatile("" : "+v"(of.vfrag[db][0]), "+v"(of.vfrag[db][1]));
    };
    if constexpr (TW == 1) {
      // (kept apart from the TW > 1 loop: a one-trip loop around the step
      // changed the register allocation of these kernels)
      fresh_offsets();
      if (tt < nkt_w) {
        if (tt < nfull)
          W::template step<false>(kc, vc, of, qreg, doreg, dqacc, C, nlse2, dlt, tt * BC, lim, hh);
        else
          W::template step<true>(kc, vc, of, qreg, doreg, dqacc, C, nlse2, dlt, tt * BC, lim, hh);
      }
    } else {
#pragma unroll
      for (int h = 0; h < TW; ++h) {
        fresh_offsets();
        const int kt = tt * TW + h;  // BC-key step
        const int eo = h * BC * D;   // its rows in the LDS tile
        if (kt < nkt_w) {
          if (kt < nfull)
            W::template step<false>(kc + eo, vc + eo, of, qreg, doreg, dqacc, C, nlse2, dlt, kt * BC, lim, hh);
          else
            W::template step<true>(kc + eo, vc + eo, of, qreg, doreg, dqacc, C, nlse2, dlt, kt * BC, lim, hh);
        }
      }
    }
    wait_vm_lds<0>();
    barrier_keep_loads();
  };
  for (int tt = 0; tt < ntt; tt += 2) {
    iteration(tt, std::integral_constant<int, 0>{});
    if (tt + 1 < ntt) iteration(tt + 1, std::integral_constant<int, 1>{});
  }

  // dQ = scale * acc: lane holds column qrow, rows d = 32 db + 8 g + 4 h + 0..3
  if (qrow < S) {
    uint16_t* row = dQ + base + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * db + 8 * g + 4 * hh;
        *reinterpret_cast<u32x2*>(row + d) = pack_bf16x4(dqacc[db][4 * g] * scale, dqacc[db][4 * g + 1] * scale,
                                                         dqacc[db][4 * g + 2] * scale, dqacc[db][4 * g + 3] * scale);
      }
    }
  }
}

template <class Cfg, int OCC, int TW = 1>
static hipError_t launch_dq_t(const BwdArgs& a, hipStream_t st) {
  const int nqt = (a.S + Cfg::BR - 1) / Cfg::BR;
  const int BH = a.B * a.H;
  prof_begin(KID_BWD_DQ, st);
  hipLaunchKernelGGL((bwd_dq_kernel<Cfg, OCC, TW>), dim3(nqt * BH), dim3(64 * Cfg::NW), 0, st, (const uint16_t*)a.Q,
                     (const uint16_t*)a.K, (const uint16_t*)a.V, (const uint16_t*)a.dO, (const uint16_t*)a.O,
                     a.LSE, a.nlse2, a.delta, (uint16_t*)a.dQ, BH, a.S, a.scale, a.scale * kLog2e, nqt, a.causal);
  prof_end(KID_BWD_DQ, st);
  return hipGetLastError();
}

// Every head dim takes the pipelined step over 64-key tiles.  Against a
// plain step (a tile's S and dP products, then its softmax, then its dQ
// product), measured in interleaved same-process runs at S = 8192, B=2,
// H=16: D = 64 0.764 against 0.781 ms non-causal (two workgroups of four
// wavefronts per CU), 0.388 against 0.395 causal; D = 256 3.208 against
// 3.346 ms non-causal (32-key tiles before), 1.644 against 1.756 causal.
// D = 128, non-causal with S >= 8192: the cooperative big tile, one
// workgroup of eight wavefronts (256 queries) per CU sharing each K / V tile
// in LDS, 64-key steps in the pipelined step, two steps per LDS tile (128
// KiB of LDS: one load issue and one barrier per 128 keys).  Otherwise two
// workgroups of four wavefronts per CU, which balance shorter and causal
// passes better.  Interleaved same-process A/B of the two (B*H*S fixed at
// 2^19, D = 128; ms, eight against four wavefronts): S = 2048 0.396 / 0.366
// non-causal, 0.231 / 0.206 causal; S = 4096 0.690 / 0.676, 0.375 / 0.360;
// S = 8192 1.300 / 1.315, 0.683 / 0.677; S = 32768 (B*H = 32) 20.21 / 20.42,
// 10.30 / 10.27.  Variants (attn_set_variant("bwd_dq", v) or
// ATTN97_DQ_VARIANT=v): 1 four wavefronts, 2 eight wavefronts, at every
// length.
static int dq_variant() { return kernel_variant(VAR_DQ); }

hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t st) {
  switch (a.D) {
    case 64: return launch_dq_t<FwdCfg<64, 64, 4, 2>, 2>(a, st);  // two workgroups (eight wavefronts) per CU
    case 128:
      if (dq_variant() == 2 || (dq_variant() == 0 && !a.causal && a.S >= 8192))
        return launch_dq_t<FwdCfg<128, 64, 8, 2>, 1, 2>(a, st);
      return launch_dq_t<FwdCfg<128, 64, 4, 2>, 2>(a, st);
    case 256: return launch_dq_t<FwdCfg<256, 64, 4, 2>, 1>(a, st);  // one workgroup per CU
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn97

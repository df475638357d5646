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
// and Kernel Pipelining Co-Design for Asymmetric Hardware Scaling".
//
// Computing S transposed (keys as MFMA rows, queries as columns) puts every
// score of one query row in one lane pair (l, l+32): the row max and row sum
// are in-lane, and the rescale of the output accumulator is a per-lane scalar.
//
// Data movement: K and V tiles are double-buffered in LDS.  The loads of tile
// j+1 are issued into registers before tile j is computed and written to the
// other LDS buffer after it, so one barrier per tile suffices.  K is stored
// row-major; V is stored transposed (d-major) with the key order permuted
// inside 16-key groups so that the V^T operand of the second product is one
// ds_read_b128 per lane.
#include "attn_kernels.hpp"
#include "device_common.hpp"

namespace attn97 {

template <int D>
struct FwdCfg {
  static constexpr int BC = (D == 64) ? 128 : (D == 128 ? 64 : 32);  // keys per tile
  static constexpr int BR = 128;                                     // queries per workgroup
  static constexpr int KRS = D + 8;                                  // K row stride (elements)
  static constexpr int VRS = BC + 8;                                 // V^T row stride (elements)
  static constexpr int NKB = BC / 32;                                // 32-key blocks per tile
  static constexpr int NKS = D / 16;                                 // reduction steps over D
  static constexpr int NDB = D / 32;                                 // 32-wide blocks of D
  static constexpr int KPT = BC * D / 8 / 256;                       // 16-byte K chunks per thread
};

template <int D, bool CAUSAL, int EXPMODE>
__global__ __launch_bounds__(256, (D == 256) ? 1 : 2) void fwd_kernel(const uint16_t* __restrict__ Q,
                                                     const uint16_t* __restrict__ K,
                                                     const uint16_t* __restrict__ V,
                                                     uint16_t* __restrict__ O,
                                                     float* __restrict__ LSE, int BH, int S,
                                                     float C, uint32_t qsign, float tau, int nqt) {
  using Cfg = FwdCfg<D>;
  constexpr int BC = Cfg::BC, BR = Cfg::BR, KRS = Cfg::KRS, VRS = Cfg::VRS;
  constexpr int NKB = Cfg::NKB, NKS = Cfg::NKS, NDB = Cfg::NDB, KPT = Cfg::KPT;
  static_assert(BC * D == 8192, "one V unit (4 keys x 8 d) per thread");

  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][BC * KRS];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2][D * VRS];

  // Heaviest causal query tiles first, all heads of one rank together; with
  // B*H a multiple of 8 every workgroup of one head lands on the same XCD.
  const int id = blockIdx.x;
  const int bh = id % BH;
  const int rank = id / BH;
  const int qt = CAUSAL ? (nqt - 1 - rank) : rank;
  const int q0 = qt * BR;
  const size_t base = (size_t)bh * (size_t)S * D;

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
    const u32x4* src = reinterpret_cast<const u32x4*>(Q + base + (size_t)qrow * D);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (qrow < S) v = src[2 * ks + hh];
      v ^= qsign;
      qreg[ks] = as_bf16x8(v);
    }
  }

  const int kend = CAUSAL ? min(S, q0 + BR) : S;
  const int nkt = (kend + BC - 1) / BC;

  // Global -> register staging of one K/V tile.
  u32x4 kst[KPT];
  u32x4 vst[4];
  const int vg = tid % (BC / 4);  // V unit: key group (4 keys) ...
  const int vc = tid / (BC / 4);  // ... and d chunk (8 values)
  auto gload = [&](int kt) {
    const int k0 = kt * BC;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int cid = i * 256 + tid;
      const int key = cid / (D / 8);
      const int c = cid % (D / 8);
      u32x4 v = {0u, 0u, 0u, 0u};
      if (k0 + key < S) v = *reinterpret_cast<const u32x4*>(K + base + (size_t)(k0 + key) * D + c * 8);
      kst[i] = v;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = k0 + 4 * vg + i;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (key < S) v = *reinterpret_cast<const u32x4*>(V + base + (size_t)key * D + vc * 8);
      vst[i] = v;
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int cid = i * 256 + tid;
      const int key = cid / (D / 8);
      const int c = cid % (D / 8);
      *reinterpret_cast<u32x4*>(&Ks[buf][key * KRS + c * 8]) = kst[i];
    }
    store_transposed_4x8(Vt[buf], VRS, vc * 8, perm_pos_of_group(vg), vst);
  };

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
  float m_run = kNegInf;  // running max, in units of log2 (scores times C)
  float l_part = 0.0f;    // this lane's partial row sum

  gload(0);
  lstore(0);
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    const int k0 = kt * BC;
    if (kt + 1 < nkt) gload(kt + 1);

    const bool active = !CAUSAL || (k0 <= qw0 + 31);  // wave-uniform
    if (active) {
      // ---- S^T = K Q^T --------------------------------------------------
      f32x16 sacc[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) sacc[kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const bf16x8 a = lds_frag(&Ks[buf][(32 * kb + c32) * KRS + 16 * ks + 8 * hh]);
          sacc[kb] = mfma32(a, qreg[ks], sacc[kb]);
        }
      }

      // ---- mask (diagonal / ragged tiles only) and row max ------------------
      const bool need_mask = (CAUSAL && (k0 + BC - 1 > qw0)) || (k0 + BC > S);
      float mx = kNegInf;
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
            const bool hide = (key >= S) || (CAUSAL && key > qrow);
            if (hide) sacc[kb][r] = kNegInf;
            mx = __builtin_fmaxf(mx, sacc[kb][r]);
          }
        }
      } else {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, sacc[kb][r]);
        }
      }
      mx = __builtin_fmaxf(mx, wave_swap_halves(mx));
      const float mxs = (mx == kNegInf) ? kNegInf : mx * C;
      const float m_new = __builtin_fmaxf(m_run, mxs);

      // ---- conditional rescale (wave-uniform decision) --------------------
      const bool grow = (m_new - m_run) > tau;  // true on the first tile (m_run = -inf)
      if (__any(grow)) {
        const float alpha = (m_new == kNegInf) ? 1.0f : exp2_native(m_run - m_new);
        m_run = m_new;
        l_part *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
      }

      // ---- P = exp2(S*C - m), row sum, bf16 pack --------------------------
      const float negm = -m_run;
      bf16x8 pb[2 * NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float e = exp2_mode<EXPMODE>(__builtin_fmaf(sacc[kb][r], C, negm), r);
          if (need_mask && sacc[kb][r] == kNegInf) e = 0.0f;
          p[r] = e;
          l_part += e;
        }
        pb[2 * kb] = to_bf16x8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
        pb[2 * kb + 1] = to_bf16x8(p[8], p[9], p[10], p[11], p[12], p[13], p[14], p[15]);
      }

      // ---- O^T += V^T P^T ---------------------------------------------------
#pragma unroll
      for (int t = 0; t < 2 * NKB; ++t) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const bf16x8 a = lds_frag(&Vt[buf][(32 * db + c32) * VRS + 16 * t + 8 * hh]);
          oacc[db] = mfma32(a, pb[t], oacc[db]);
        }
      }
    }

    if (kt + 1 < nkt) lstore(buf ^ 1);
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
template <int D, bool CAUSAL, int EXPMODE>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t st) {
  const int nqt = (a.S + FwdCfg<D>::BR - 1) / FwdCfg<D>::BR;
  const int BH = a.B * a.H;
  dim3 grid(nqt * BH), block(256);
  prof_begin(KID_FWD, st);
  hipLaunchKernelGGL((fwd_kernel<D, CAUSAL, EXPMODE>), grid, block, 0, st,
                     (const uint16_t*)a.Q, (const uint16_t*)a.K, (const uint16_t*)a.V,
                     (uint16_t*)a.O, a.LSE, BH, a.S, a.C, a.qsign, a.tau, nqt);
  prof_end(KID_FWD, st);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
static hipError_t launch_fwd_e(const FwdArgs& a, hipStream_t st) {
  switch (a.exp_mode) {
    case 1: return launch_fwd_t<D, CAUSAL, 1>(a, st);
    case 2: return launch_fwd_t<D, CAUSAL, 2>(a, st);
    default: return launch_fwd_t<D, CAUSAL, 0>(a, st);
  }
}

template <int D>
static hipError_t launch_fwd_c(const FwdArgs& a, hipStream_t st) {
  return a.causal ? launch_fwd_e<D, true>(a, st) : launch_fwd_e<D, false>(a, st);
}

hipError_t launch_fwd(const FwdArgs& a, hipStream_t st) {
  switch (a.D) {
    case 64: return launch_fwd_c<64>(a, st);
    case 128: return launch_fwd_c<128>(a, st);
    case 256: return launch_fwd_c<256>(a, st);
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

// attn_bwd.hip - backward pass of exact attention on gfx950 (dQ by atomics).
//
// The forward pass stored only O and the row log-sum-exp, so the backward
// pass recomputes the probabilities from them:
//
//   Delta_i = sum_d dO_id O_id                       (bwd_pre_kernel)
//   P  = exp2(S * scale*log2e - LSE*log2e),  S = Q K^T
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
#include "attn_kernels.hpp"
#include "device_common.hpp"

namespace attn97 {

template <int D>
struct BwdCfg {
  static constexpr int NW = 4;                     // wavefronts per workgroup
  static constexpr int BK = 32 * NW;               // keys per workgroup
  static constexpr int BQ = 64;                    // queries per tile
  static constexpr int NQB = BQ / 32;              // 32-query blocks per tile
  static constexpr int NKS = D / 16;               // reduction steps over D
  static constexpr int NDB = D / 32;               // 32-wide blocks of D
  static constexpr int QRS = D + 8;                // row stride of Qs / dOs (elements)
  static constexpr int TRS = BQ + 8;               // row stride of Qt / dOt
  static constexpr int SRS = BK + 8;               // row stride of dSs / Kt
  static constexpr int NDQ = NQB * NDB / NW;       // dQ blocks per wavefront
  static constexpr int UNITS = (BQ / 4) * (D / 8); // 4x8 staging units per tensor
  static constexpr int UPT = 2 * UNITS / 256;      // staging units per thread (Q and dO)
  static_assert(NDQ >= 1 && NQB * NDB == NDQ * NW, "dQ blocks split evenly");
  static_assert(2 * UNITS % 256 == 0 && UPT >= 1, "staging units split evenly");
};

template <int D>
struct BwdSmem {
  using Cfg = BwdCfg<D>;
  uint16_t Qs[Cfg::BQ * Cfg::QRS];
  uint16_t dOs[Cfg::BQ * Cfg::QRS];
  uint16_t Qt[D * Cfg::TRS];
  uint16_t dOt[D * Cfg::TRS];
  uint16_t dSs[Cfg::BQ * Cfg::SRS];
  uint16_t Kt[D * Cfg::SRS];
  float lse2s[Cfg::BQ];
  float dlts[Cfg::BQ];
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

// One query tile against one wavefront's 32 keys: S = Q K^T and dP = dO V^T,
// P = exp2(S c - LSE log2e), dS = P (dP - Delta), dS to LDS (queries as rows)
// for the dQ product, then dV += P^T dO and dK += dS^T Q.  MASK selects the
// diagonal / ragged path; the interior runs without any masking.
template <int D, bool CAUSAL, bool MASK>
__device__ __forceinline__ void bwd_tile(BwdSmem<D>& sm, const bf16x8 (&kreg)[D / 16],
                                         const bf16x8 (&vreg)[D / 16], f32x16 (&dk)[D / 32],
                                         f32x16 (&dv)[D / 32], int q0, int key, int S, float C, int c32,
                                         int hh, int dsw) {
  using Cfg = BwdCfg<D>;
  constexpr int NQB = Cfg::NQB, NKS = Cfg::NKS, NDB = Cfg::NDB, QRS = Cfg::QRS, TRS = Cfg::TRS,
                SRS = Cfg::SRS;
  const bool odd = c32 & 1;
  bf16x8 pb[2 * NQB], dsb[2 * NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    f32x16 sacc = f32x16{}, dpacc = f32x16{};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      sacc = mfma32(lds_frag(&sm.Qs[(32 * qb + c32) * QRS + 16 * ks + 8 * hh]), kreg[ks], sacc);
      dpacc = mfma32(lds_frag(&sm.dOs[(32 * qb + c32) * QRS + 16 * ks + 8 * hh]), vreg[ks], dpacc);
    }
    float p[16], ds[16];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int qr = 32 * qb + 8 * g + 4 * hh;  // tile row of register 4g
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(&sm.lse2s[qr]);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(&sm.dlts[qr]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * g + e;
        float pv = exp2_native(__builtin_fmaf(sacc[r], C, -l4[e]));
        if (MASK) {
          if (key >= S || (CAUSAL && key > q0 + qr + e)) pv = 0.0f;
        }
        p[r] = pv;
        ds[r] = pv * (dpacc[r] - d4[e]);
      }
    }
    pb[2 * qb] = to_bf16x8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
    pb[2 * qb + 1] = to_bf16x8(p[8], p[9], p[10], p[11], p[12], p[13], p[14], p[15]);
    dsb[2 * qb] = to_bf16x8(ds[0], ds[1], ds[2], ds[3], ds[4], ds[5], ds[6], ds[7]);
    dsb[2 * qb + 1] = to_bf16x8(ds[8], ds[9], ds[10], ds[11], ds[12], ds[13], ds[14], ds[15]);
    // dS to LDS with queries as rows.  Lanes l and l^1 hold adjacent keys; for
    // rows (r, r+1) the even lane writes row r and the odd lane row r+1, each
    // as one 32-bit pair of adjacent keys (dsw already holds the odd lane's
    // one-row offset and the even key column).
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float recv = swap_lane_pair(odd ? ds[r] : ds[r + 1]);
      const float lo = odd ? recv : ds[r];
      const float hi = odd ? ds[r + 1] : recv;
      const int row = 32 * qb + 8 * (r >> 2) + 4 * hh + (r & 3);
      *reinterpret_cast<uint32_t*>(&sm.dSs[row * SRS + dsw]) = pack_bf16x2(lo, hi);
    }
  }
#pragma unroll
  for (int t = 0; t < 2 * NQB; ++t) {
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      dv[db] = mfma32(pb[t], lds_frag(&sm.dOt[(32 * db + c32) * TRS + 16 * t + 8 * hh]), dv[db]);
      dk[db] = mfma32(dsb[t], lds_frag(&sm.Qt[(32 * db + c32) * TRS + 16 * t + 8 * hh]), dk[db]);
    }
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_main_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ delta,
    float* __restrict__ dq32, uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int BH, int S,
    float scale, float C) {
  using Cfg = BwdCfg<D>;
  constexpr int BK = Cfg::BK, BQ = Cfg::BQ, NKS = Cfg::NKS, NDB = Cfg::NDB, QRS = Cfg::QRS,
                TRS = Cfg::TRS, SRS = Cfg::SRS, NDQ = Cfg::NDQ, UNITS = Cfg::UNITS, UPT = Cfg::UPT;

  __shared__ __attribute__((aligned(16))) BwdSmem<D> sm;

  const int id = blockIdx.x;
  const int bh = id % BH;
  const int ktile = id / BH;  // causal: lowest keys (most work) first
  const int k0 = ktile * BK;
  const size_t base = (size_t)bh * (size_t)S * D;
  const uint16_t* Qh = Q + base;
  const uint16_t* Kh = K + base;
  const uint16_t* Vh = V + base;
  const uint16_t* dOh = dO + base;
  const float* LSEh = LSE + (size_t)bh * S;
  const float* dlth = delta + (size_t)bh * S;
  float* dqh = dq32 + base;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int hh = lane >> 5;
  const int c32 = lane & 31;
  const int kw0 = k0 + 32 * wave;  // first key of this wavefront
  const int key = kw0 + c32;       // this lane's key (MFMA column)
  const int keyc = min(key, S - 1);

  // K^T / V^T operands of S = Q K^T and dP = dO V^T: lane holds row `key`.
  // Rows past the end are clamped (finite data); their P is masked to zero.
  bf16x8 kreg[NKS], vreg[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const uint32_t off = (uint32_t)keyc * D + 16 * ks + 8 * hh;
    kreg[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(Kh + off));
    vreg[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(Vh + off));
  }

  // K transposed into LDS for the dQ product (B operand, keys permuted).
  for (int u = tid; u < (BK / 4) * (D / 8); u += 256) {
    const int g = u % (BK / 4);
    const int c = u / (BK / 4);
    u32x4 rows[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t kk = min(k0 + 4 * g + i, S - 1);
      rows[i] = *reinterpret_cast<const u32x4*>(Kh + kk * D + 8 * c);
    }
    store_transposed_4x8(sm.Kt, SRS, 8 * c, perm_pos_of_group(g), rows);
  }

  // Staging of one query tile through registers: UPT units of 4 rows x 8
  // columns of Q or dO per thread; threads 0..BQ-1 also take LSE and Delta.
  u32x4 srows[UPT][4];
  float s_lse = 0.0f, s_dlt = 0.0f;
  auto stage = [&](int qt) {
    const int q0 = qt * BQ;
#pragma unroll
    for (int j = 0; j < UPT; ++j) {
      const int u = tid + 256 * j;
      const uint16_t* src = (u < UNITS) ? Qh : dOh;
      const int lu = u % UNITS;
      const int g = lu % (BQ / 4);
      const int c = lu / (BQ / 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t q = min(q0 + 4 * g + i, S - 1);
        srows[j][i] = *reinterpret_cast<const u32x4*>(src + q * D + 8 * c);
      }
    }
    if (tid < BQ) {
      const int q = q0 + tid;
      s_lse = (q < S) ? LSEh[q] * kLog2e : __builtin_huge_valf();  // rows past the end: P = 0
      s_dlt = (q < S) ? dlth[q] : 0.0f;
    }
  };
  auto commit = [&]() {
#pragma unroll
    for (int j = 0; j < UPT; ++j) {
      const int u = tid + 256 * j;
      const bool isq = u < UNITS;
      const int lu = u % UNITS;
      const int g = lu % (BQ / 4);
      const int c = lu / (BQ / 4);
      uint16_t* rowdst = isq ? sm.Qs : sm.dOs;
      uint16_t* trdst = isq ? sm.Qt : sm.dOt;
#pragma unroll
      for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(rowdst + (4 * g + i) * QRS + 8 * c) = srows[j][i];
      store_transposed_4x8(trdst, TRS, 8 * c, perm_pos_of_group(g), srows[j]);
    }
    if (tid < BQ) {
      sm.lse2s[tid] = s_lse;
      sm.dlts[tid] = s_dlt;
    }
  };

  f32x16 dk[NDB], dv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }

  const int nqt = (S + BQ - 1) / BQ;
  const int qt0 = CAUSAL ? (k0 / BQ) : 0;
  stage(qt0);
  commit();
  __syncthreads();

  // This lane's dS write column: the even key of its lane pair, one row down
  // for the odd lane.
  const int dsw = (c32 & 1) * SRS + (perm_pos_of_row(32 * wave + c32) & ~1);

  for (int qt = qt0; qt < nqt; ++qt) {
    const int q0 = qt * BQ;
    if (qt + 1 < nqt) stage(qt + 1);

    const bool active = !CAUSAL || (q0 + BQ - 1 >= kw0);  // wave-uniform
    if (active) {
      const bool need_mask = (CAUSAL && q0 < kw0 + 31) || (kw0 + 32 > S);
      if (need_mask)
        bwd_tile<D, CAUSAL, true>(sm, kreg, vreg, dk, dv, q0, key, S, C, c32, hh, dsw);
      else
        bwd_tile<D, CAUSAL, false>(sm, kreg, vreg, dk, dv, q0, key, S, C, c32, hh, dsw);
    } else {
#pragma unroll
      for (int r = 0; r < 2 * BQ / 4; r += 2) {
        const int row = 32 * (r >> 4) + 8 * ((r & 15) >> 2) + 4 * hh + (r & 3);
        *reinterpret_cast<uint32_t*>(&sm.dSs[row * SRS + dsw]) = 0u;
      }
    }
    __syncthreads();  // dSs complete; Q/dO tile no longer read

    if (qt + 1 < nqt) commit();

    // ---- dQ[q, d] += scale * dS K over the workgroup's keys ---------------
#pragma unroll
    for (int j = 0; j < NDQ; ++j) {
      const int bi = wave * NDQ + j;
      const int qb = bi / NDB;
      const int db = bi % NDB;
      f32x16 acc0 = f32x16{}, acc1 = f32x16{};
#pragma unroll
      for (int t = 0; t < BK / 16; t += 2) {
        acc0 = mfma32(lds_frag(&sm.dSs[(32 * qb + c32) * SRS + 16 * t + 8 * hh]),
                      lds_frag(&sm.Kt[(32 * db + c32) * SRS + 16 * t + 8 * hh]), acc0);
        acc1 = mfma32(lds_frag(&sm.dSs[(32 * qb + c32) * SRS + 16 * t + 16 + 8 * hh]),
                      lds_frag(&sm.Kt[(32 * db + c32) * SRS + 16 * t + 16 + 8 * hh]), acc1);
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
    __syncthreads();  // dSs read; next Q/dO tile visible
  }

  // ---- epilogue: dK = scale * acc, dV = acc (bf16) -------------------------
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int d = 32 * db + c32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kk = kw0 + 8 * (r >> 2) + 4 * hh + (r & 3);
      if (kk < S) {
        dK[base + (size_t)kk * D + d] = __builtin_bit_cast(uint16_t, (__bf16)(dk[db][r] * scale));
        dV[base + (size_t)kk * D + d] = __builtin_bit_cast(uint16_t, (__bf16)dv[db][r]);
      }
    }
  }
}

// Delta_i = sum_d dO_id O_id (fp32) and zero the fp32 dQ accumulator.
// D/8 lanes share one row; each lane takes eight columns.
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const uint16_t* __restrict__ O,
                                                      const uint16_t* __restrict__ dO,
                                                      float* __restrict__ delta,
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
  if (c == 0 && row < rows) delta[row] = acc;
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

bool bwd_supported(int D) { return D == 64 || D == 128; }

template <int D, bool CAUSAL>
static hipError_t launch_main_t(const BwdArgs& a, hipStream_t st) {
  const int BH = a.B * a.H;
  const int nkt = (a.S + BwdCfg<D>::BK - 1) / BwdCfg<D>::BK;
  prof_begin(KID_BWD_MAIN, st);
  hipLaunchKernelGGL((bwd_main_kernel<D, CAUSAL>), dim3(nkt * BH), dim3(256), 0, st,
                     (const uint16_t*)a.Q, (const uint16_t*)a.K, (const uint16_t*)a.V,
                     (const uint16_t*)a.dO, a.LSE, a.delta, a.dq32, (uint16_t*)a.dK,
                     (uint16_t*)a.dV, BH, a.S, a.scale, a.scale * kLog2e);
  prof_end(KID_BWD_MAIN, st);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_pre_t(const BwdArgs& a, hipStream_t st) {
  const long rows = (long)a.B * a.H * a.S;
  const long threads = rows * (D / 8);
  prof_begin(KID_BWD_PRE, st);
  hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st,
                     (const uint16_t*)a.O, (const uint16_t*)a.dO, a.delta, a.dq32, rows);
  prof_end(KID_BWD_PRE, st);
  return hipGetLastError();
}

hipError_t launch_bwd_atomic(const BwdArgs& a, hipStream_t st) {
  hipError_t e;
  switch (a.D) {
    case 64: e = launch_pre_t<64>(a, st); break;
    case 128: e = launch_pre_t<128>(a, st); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  switch (a.D * 2 + (a.causal ? 1 : 0)) {
    case 128: e = launch_main_t<64, false>(a, st); break;
    case 129: e = launch_main_t<64, true>(a, st); break;
    case 256: e = launch_main_t<128, false>(a, st); break;
    case 257: e = launch_main_t<128, true>(a, st); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  const long n8 = (long)a.B * a.H * a.S * a.D / 8;
  prof_begin(KID_DQ_CONVERT, st);
  hipLaunchKernelGGL(dq_convert_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st,
                     (const float*)a.dq32, (uint16_t*)a.dQ, n8);
  prof_end(KID_DQ_CONVERT, st);
  return hipGetLastError();
}

}  // namespace attn97

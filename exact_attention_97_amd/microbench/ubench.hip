// ubench.hip - pipe ceilings of the MI355X (gfx950) compute unit that the
// attention kernels are designed against: matrix-core throughput per MFMA
// shape, VALU and transcendental issue cost, the overlap of a wavefront's
// own MFMAs with its VALU work, LDS read bandwidth for the read forms the
// kernels use, and the rate and placement of fp32 atomic adds.  None of these figures are on the pages; they are measured.
//
// Each kernel reads the shader clock (s_memtime) in every wavefront around
// its timed loop, so per-instruction costs are in core clock cycles; HIP
// events around the whole-chip MFMA launches give achieved TFLOP/s and the
// effective clock under that load.
//
// Build: hipcc --offload-arch=gfx950 -O3 -std=c++17
//          -Xclang -target-feature -Xclang -packed-fp32-ops
//          -I exact_attention_97_amd/csrc ubench.hip -o ubench
// (exact_attention_97_amd/build_lib.py builds it as microbench/ubench).
// Run: ./ubench   prints one markdown table per section;
//      ./ubench atomic   only the atomic section (for counter runs).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "device_common.hpp"

namespace ub {
using namespace attn97;

typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef short s16x4v __attribute__((ext_vector_type(4)));
typedef int i32x8v __attribute__((ext_vector_type(8)));

constexpr int kBlocks = 256;  // one workgroup per CU
constexpr int kMaxWaves = 16;

#define UB_CHECK(x)                                                                  \
  do {                                                                               \
    hipError_t e_ = (x);                                                             \
    if (e_ != hipSuccess) {                                                          \
      fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #x, hipGetErrorString(e_)); \
      exit(1);                                                                       \
    }                                                                                \
  } while (0)

// ---- matrix core ----------------------------------------------------------
// SHAPE 0: v_mfma_f32_32x32x16_bf16 (32768 flop), 1: v_mfma_f32_16x16x32_bf16
// (16384 flop), 2: v_mfma_scale_f32_32x32x64_f8f6f4 with E4M3 operands
// (131072 flop), four independent accumulator chains per wavefront; 3 and 4:
// v_mfma_f32_32x32x16_bf16 with one chain (each MFMA accumulates onto the
// previous one's result) and with two chains.
template <int SHAPE>
__global__ __launch_bounds__(1024) void k_mfma(const float* __restrict__ in, float* __restrict__ out,
                                               long long* __restrict__ cyc, int iters) {
  const int tid = threadIdx.x, lane = tid & 63;
  const float x = in[lane];
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(x + i);
    b[i] = (__bf16)(x - i);
  }
  i32x8v a8, b8;
  for (int i = 0; i < 8; ++i) {
    a8[i] = 0x38383838 + i;
    b8[i] = 0x30303030 + lane;
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  f32x4v d0 = {}, d1 = {}, d2 = {}, d3 = {};
  __syncthreads();
  const long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if constexpr (SHAPE == 0) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
      } else if constexpr (SHAPE == 1) {
        d0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, d0, 0, 0, 0);
        d1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, d1, 0, 0, 0);
        d2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, d2, 0, 0, 0);
        d3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, d3, 0, 0, 0);
      } else if constexpr (SHAPE == 3) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
      } else if constexpr (SHAPE == 4) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
      } else {
        c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c0, 0, 0, 0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c1, 0, 0, 0, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c2, 0, 0, 0, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c3, 0, 0, 0, 0, 0, 0);
      }
    }
  }
  const long long t1 = __builtin_amdgcn_s_memtime();
  float s = 0.f;
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  for (int i = 0; i < 4; ++i) s += d0[i] + d1[i] + d2[i] + d3[i];
  out[blockIdx.x * blockDim.x + tid] = s;
  if (lane == 0) {
    cyc[2 * (blockIdx.x * kMaxWaves + (tid >> 6))] = t0;
    cyc[2 * (blockIdx.x * kMaxWaves + (tid >> 6)) + 1] = t1;
  }
}

// ---- VALU and transcendental issue ----------------------------------------
// OP 0: v_fma_f32, 1: v_exp_f32, 2: the degree-3 polynomial exp2 of the
// forward kernel (one element = range reduction, polynomial, ldexp).  Eight
// independent chains, so the cost is issue, not latency.
template <int OP>
__global__ __launch_bounds__(1024) void k_valu(const float* __restrict__ in, float* __restrict__ out,
                                               long long* __restrict__ cyc, int iters) {
  const int tid = threadIdx.x, lane = tid & 63;
  float x[8];
  for (int i = 0; i < 8; ++i) x[i] = in[(lane + i) & 63] - 1.0f;
  const float m = in[1] * 0.25f + 0.5f, k = in[2] * 0.125f - 0.25f;
  __syncthreads();
  const long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if constexpr (OP == 0) x[i] = __builtin_fmaf(x[i], m, k);
        else if constexpr (OP == 1) x[i] = exp2_native(x[i]) - 1.5f;
        else x[i] = exp2_poly(x[i]) - 1.5f;
      }
    }
  }
  const long long t1 = __builtin_amdgcn_s_memtime();
  float s = 0.f;
  for (int i = 0; i < 8; ++i) s += x[i];
  out[blockIdx.x * blockDim.x + tid] = s;
  if (lane == 0) {
    cyc[2 * (blockIdx.x * kMaxWaves + (tid >> 6))] = t0;
    cyc[2 * (blockIdx.x * kMaxWaves + (tid >> 6)) + 1] = t1;
  }
}

// ---- a wavefront's MFMAs with its own VALU work ----------------------------
// Per step: one 32x32x16 MFMA (two chains alternate), NV independent fp32
// FMAs and NE exponentials; the scheduling barriers keep that order.
template <int NV, int NE>
__global__ __launch_bounds__(256) void k_overlap(const float* __restrict__ in, float* __restrict__ out,
                                                 long long* __restrict__ cyc, int iters) {
  const int tid = threadIdx.x, lane = tid & 63;
  float x[8];
  for (int i = 0; i < 8; ++i) x[i] = in[(lane + 3 * i) & 63] - 1.0f;
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)in[(lane + i) & 63];
    b[i] = (__bf16)in[(2 * lane + i) & 63];
  }
  f32x16 c0 = {}, c1 = {};
  const float m = in[1] * 0.25f + 0.5f, k = in[2] * 0.125f - 0.25f;
  __syncthreads();
  const long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (u & 1) c1 = mfma32(a, b, c1);
      else c0 = mfma32(a, b, c0);
#pragma unroll
      for (int v = 0; v < NV; ++v) x[v & 7] = __builtin_fmaf(x[v & 7], m, k);
#pragma unroll
      for (int e = 0; e < NE; ++e) x[(e + 4) & 7] = exp2_native(x[(e + 4) & 7]) - 1.5f;
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if constexpr (NV + NE > 0) __builtin_amdgcn_sched_group_barrier(0x002, NV + NE, 0);
    }
  }
  const long long t1 = __builtin_amdgcn_s_memtime();
  float s = 0.f;
  for (int i = 0; i < 8; ++i) s += x[i];
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i];
  out[blockIdx.x * blockDim.x + tid] = s;
  if (lane == 0) {
    cyc[2 * (blockIdx.x * kMaxWaves + (tid >> 6))] = t0;
    cyc[2 * (blockIdx.x * kMaxWaves + (tid >> 6)) + 1] = t1;
  }
}

// ---- LDS reads -------------------------------------------------------------
// A 64 KB buffer of 256-byte rows.  KIND 0: ds_read_b128, lane l reading row
// l%32 at a 16-byte chunk XOR-swizzled by the row (the kernels' tile layout:
// no bank conflicts); 1: ds_read_b128 with the chunk not swizzled (32 lanes on
// one 16-byte column of 32 rows); 2: ds_read_b64_tr_b16 (the transposing read
// of the P V and dS K products), swizzled.  Sixteen reads per iteration, all
// in flight before the data is used.
template <int KIND>
__global__ __launch_bounds__(1024) void k_lds(float* __restrict__ out, long long* __restrict__ cyc, int iters) {
  __shared__ __attribute__((aligned(1024))) uint16_t buf[32768];
  const int tid = threadIdx.x, lane = tid & 63;
  for (int i = tid; i < 32768; i += blockDim.x) buf[i] = (uint16_t)(i * 7);
  __syncthreads();
  const uint32_t row = (uint32_t)(lane & 31);
  const uint32_t chunk = (uint32_t)((lane >> 5) + 2 * ((tid >> 6) & 7));
  uint32_t base = row * 256u + (KIND == 1 ? (chunk & 15u) : ((chunk ^ row) & 15u)) * 16u;
  u32x4 acc = {0, 0, 0, 0};
  const long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
    asm volatile("" : "+v"(base));  // a fresh address each iteration: nothing is hoisted
    const uint32_t off = (uint32_t)(it & 3) * 2048u;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const uint32_t a = (base + (uint32_t)(k & 7) * 8192u + off + (uint32_t)(k >> 3) * 1024u) & 65535u;
      const char* p = reinterpret_cast<const char*>(buf) + a;
      if constexpr (KIND == 2) {
        const s16x4v r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4v*)(p));
        acc[k & 3] += (uint32_t)(uint16_t)r[0] | ((uint32_t)(uint16_t)r[1] << 16);
        acc[(k + 1) & 3] += (uint32_t)(uint16_t)r[2] | ((uint32_t)(uint16_t)r[3] << 16);
      } else {
        acc += *reinterpret_cast<const u32x4*>(p);
      }
    }
  }
  const long long t1 = __builtin_amdgcn_s_memtime();
  out[blockIdx.x * blockDim.x + tid] = (float)(acc[0] ^ acc[1] ^ acc[2] ^ acc[3]);
  if (lane == 0) {
    cyc[2 * (blockIdx.x * kMaxWaves + (tid >> 6))] = t0;
    cyc[2 * (blockIdx.x * kMaxWaves + (tid >> 6)) + 1] = t1;
  }
}

// ---- fp32 atomic adds -----------------------------------------------------
// No-return buffer atomic adds of 1.0 into an array of 8 regions of 64 K
// floats (2 MiB): workgroup b adds into region b % 8 (pattern 0) or
// (b / 8) % 8 (pattern 1), 256 adds per lane at addresses spread over the
// region.  With workgroups dispatched to the eight XCDs in turn, pattern 0
// keeps each region's adds on one XCD (its L2) and pattern 1 sends every
// region's adds from all of them.  SC1 sets the instruction's sc1 bit (the
// device-scope form).  Every workgroup records the XCD it ran on
// (HW_REG_XCC_ID), so the host checks the dispatch order and the sums.
constexpr int kAtomRegion = 65536, kAtomBlocks = 4096, kAtomIters = 256;
template <int SC1>
__global__ __launch_bounds__(256) void k_atomic(float* __restrict__ acc, int* __restrict__ xcc, int pattern) {
  const int b = blockIdx.x, t = threadIdx.x;
  const int region = pattern == 0 ? (b & 7) : ((b >> 3) & 7);
  if (t == 0) {
    int id;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(id));
    xcc[b] = id & 0xffff;
  }
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(acc + (size_t)region * kAtomRegion, (short)0, kAtomRegion * 4, 0x00020000);
  for (int it = 0; it < kAtomIters; ++it) {
    const int i = (t + it * 256 + b * 97) & (kAtomRegion - 1);
    __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(1.0f, rs, i * 4, 0, SC1 ? 16 : 0);
  }
}

// ---- host ------------------------------------------------------------------
struct Bufs {
  float* in;
  float* out;
  long long* cyc;
};

// Mean over the workgroups of the span from the first wavefront's start to
// the last one's end (shader clock cycles): with several wavefronts per SIMD
// their timed loops overlap, and the span is the time the SIMD spent on all
// of them.
static double avg_cycles(const Bufs& b, int waves) {
  static long long h[2 * kBlocks * kMaxWaves];
  UB_CHECK(hipMemcpy(h, b.cyc, sizeof(long long) * 2 * kBlocks * kMaxWaves, hipMemcpyDeviceToHost));
  double s = 0;
  for (int i = 0; i < kBlocks; ++i) {
    long long lo = h[2 * (i * kMaxWaves)], hi = h[2 * (i * kMaxWaves) + 1];
    for (int w = 1; w < waves; ++w) {
      lo = h[2 * (i * kMaxWaves + w)] < lo ? h[2 * (i * kMaxWaves + w)] : lo;
      hi = h[2 * (i * kMaxWaves + w) + 1] > hi ? h[2 * (i * kMaxWaves + w) + 1] : hi;
    }
    s += (double)(hi - lo);
  }
  return s / kBlocks;
}

template <class F>
static float time_ms(F launch) {
  hipEvent_t e0, e1;
  UB_CHECK(hipEventCreate(&e0));
  UB_CHECK(hipEventCreate(&e1));
  launch();  // warm-up
  UB_CHECK(hipEventRecord(e0, 0));
  launch();
  UB_CHECK(hipEventRecord(e1, 0));
  UB_CHECK(hipEventSynchronize(e1));
  float ms = 0.f;
  UB_CHECK(hipEventElapsedTime(&ms, e0, e1));
  UB_CHECK(hipEventDestroy(e0));
  UB_CHECK(hipEventDestroy(e1));
  return ms;
}

template <int SHAPE>
static void mfma_row(const Bufs& b, const char* name, double flop, int waves_per_simd) {
  const int iters = 2048, nt = 256 * waves_per_simd;
  const float ms = time_ms([&] {
    hipLaunchKernelGGL((k_mfma<SHAPE>), dim3(kBlocks), dim3(nt), 0, 0, b.in, b.out, b.cyc, iters);
  });
  UB_CHECK(hipGetLastError());
  const double cyc = avg_cycles(b, nt / 64);
  const double n = (double)iters * 16;  // MFMAs per wavefront
  const double total = flop * n * kBlocks * (nt / 64);
  printf("| %s | %d | %.2f | %.1f | %.2f |\n", name, waves_per_simd, cyc / (n * waves_per_simd), total / (ms * 1e-3) / 1e12,
         cyc / (ms * 1e-3) / 1e9);
}

template <int OP>
static void valu_row(const Bufs& b, const char* name, int waves_per_simd) {
  const int iters = 1024, nt = 256 * waves_per_simd;
  hipLaunchKernelGGL((k_valu<OP>), dim3(kBlocks), dim3(nt), 0, 0, b.in, b.out, b.cyc, iters);
  hipLaunchKernelGGL((k_valu<OP>), dim3(kBlocks), dim3(nt), 0, 0, b.in, b.out, b.cyc, iters);
  UB_CHECK(hipDeviceSynchronize());
  const double cyc = avg_cycles(b, nt / 64);
  printf("| %s | %d | %.2f |\n", name, waves_per_simd, cyc / ((double)iters * 32 * waves_per_simd));
}

template <int NV, int NE>
static void overlap_row(const Bufs& b) {
  const int iters = 2048;
  hipLaunchKernelGGL((k_overlap<NV, NE>), dim3(kBlocks), dim3(256), 0, 0, b.in, b.out, b.cyc, iters);
  hipLaunchKernelGGL((k_overlap<NV, NE>), dim3(kBlocks), dim3(256), 0, 0, b.in, b.out, b.cyc, iters);
  UB_CHECK(hipDeviceSynchronize());
  const double cyc = avg_cycles(b, 4);
  printf("| %d | %d | %.2f |\n", NV, NE, cyc / ((double)iters * 8));
}

template <int KIND>
static void lds_row(const Bufs& b, const char* name, int waves) {
  const int iters = 2048, nt = 64 * waves;
  hipLaunchKernelGGL((k_lds<KIND>), dim3(kBlocks), dim3(nt), 0, 0, b.out, b.cyc, iters);
  hipLaunchKernelGGL((k_lds<KIND>), dim3(kBlocks), dim3(nt), 0, 0, b.out, b.cyc, iters);
  UB_CHECK(hipDeviceSynchronize());
  const double cyc = avg_cycles(b, waves);
  const double bytes = (double)iters * 16 * waves * 64 * (KIND == 2 ? 8 : 16);
  printf("| %s | %d | %.1f |\n", name, waves, bytes / cyc);
}

template <int SC1>
static void atomic_row(float* acc, int* xcc, const char* name, int pattern) {
  const size_t n = (size_t)8 * kAtomRegion;
  UB_CHECK(hipMemset(acc, 0, n * sizeof(float)));
  UB_CHECK(hipDeviceSynchronize());
  hipEvent_t e0, e1;
  UB_CHECK(hipEventCreate(&e0));
  UB_CHECK(hipEventCreate(&e1));
  UB_CHECK(hipEventRecord(e0, 0));
  hipLaunchKernelGGL((k_atomic<SC1>), dim3(kAtomBlocks), dim3(256), 0, 0, acc, xcc, pattern);
  UB_CHECK(hipEventRecord(e1, 0));
  UB_CHECK(hipEventSynchronize(e1));
  UB_CHECK(hipGetLastError());
  float ms = 0.f;
  UB_CHECK(hipEventElapsedTime(&ms, e0, e1));
  UB_CHECK(hipEventDestroy(e0));
  UB_CHECK(hipEventDestroy(e1));
  static float h[8 * kAtomRegion];
  static int x[kAtomBlocks];
  UB_CHECK(hipMemcpy(h, acc, n * sizeof(float), hipMemcpyDeviceToHost));
  UB_CHECK(hipMemcpy(x, xcc, sizeof(x), hipMemcpyDeviceToHost));
  double sum = 0;
  for (size_t i = 0; i < n; ++i) sum += h[i];
  const double adds = (double)kAtomBlocks * 256 * kAtomIters;
  int rr = 0;
  for (int i = 0; i < kAtomBlocks; ++i) rr += x[i] == (i & 7);
  printf("| %s | %s | %.3f | %.1f | %s | %d of %d |\n", name,
         pattern == 0 ? "each region from one XCD" : "each region from all XCDs", ms, adds / (ms * 1e-3) / 1e9,
         sum == adds ? "exact" : "LOST", rr, kAtomBlocks);
}

static void atomic_section() {
  float* acc;
  int* xcc;
  UB_CHECK(hipMalloc(&acc, (size_t)8 * kAtomRegion * sizeof(float)));
  UB_CHECK(hipMalloc(&xcc, kAtomBlocks * sizeof(int)));
  printf("\n## fp32 atomic adds (no return, 2 MiB target)\n\n");
  printf("| instruction | pattern | ms | G adds/s | sum | workgroups on XCD (id mod 8) |\n|---|---|---|---|---|---|\n");
  for (int p = 0; p < 2; ++p) {
    atomic_row<0>(acc, xcc, "buffer_atomic_add_f32", p);
    atomic_row<1>(acc, xcc, "buffer_atomic_add_f32 sc1", p);
  }
  UB_CHECK(hipFree(acc));
  UB_CHECK(hipFree(xcc));
}

}  // namespace ub

int main(int argc, char** argv) {
  using namespace ub;
  hipDeviceProp_t prop;
  UB_CHECK(hipGetDeviceProperties(&prop, 0));
  printf("device: %s (%s), %d CUs, max clock %.0f MHz\n\n", prop.name, prop.gcnArchName, prop.multiProcessorCount,
         prop.clockRate / 1000.0);
  if (argc > 1 && argv[1][0] == 'a') {  // "atomic": only the atomic section (for counter runs)
    atomic_section();
    return 0;
  }
  Bufs b;
  UB_CHECK(hipMalloc(&b.in, 64 * sizeof(float)));
  UB_CHECK(hipMalloc(&b.out, kBlocks * 1024 * sizeof(float)));
  UB_CHECK(hipMalloc(&b.cyc, 2 * kBlocks * kMaxWaves * sizeof(long long)));
  float hin[64];
  for (int i = 0; i < 64; ++i) hin[i] = 0.01f * (float)(i % 13) - 0.05f;
  UB_CHECK(hipMemcpy(b.in, hin, sizeof(hin), hipMemcpyHostToDevice));

  printf("## Matrix core (4 independent chains per wavefront, one workgroup per CU)\n\n");
  printf("| instruction | waves/SIMD | cycles per MFMA per SIMD | chip TFLOP/s | clock GHz (memtime / event time) |\n|---|---|---|---|---|\n");
  mfma_row<0>(b, "v_mfma_f32_32x32x16_bf16", 32768.0, 1);
  mfma_row<0>(b, "v_mfma_f32_32x32x16_bf16", 32768.0, 2);
  mfma_row<1>(b, "v_mfma_f32_16x16x32_bf16", 16384.0, 1);
  mfma_row<1>(b, "v_mfma_f32_16x16x32_bf16", 16384.0, 2);
  mfma_row<2>(b, "v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3)", 131072.0, 1);
  mfma_row<2>(b, "v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3)", 131072.0, 2);
  mfma_row<3>(b, "v_mfma_f32_32x32x16_bf16, one dependent chain", 32768.0, 1);
  mfma_row<4>(b, "v_mfma_f32_32x32x16_bf16, two chains", 32768.0, 1);

  printf("\n## VALU issue (8 independent chains per wavefront)\n\n");
  printf("| operation | waves/SIMD | cycles per wavefront instruction (element for the polynomial) per SIMD |\n|---|---|---|\n");
  valu_row<0>(b, "v_fma_f32", 1);
  valu_row<0>(b, "v_fma_f32", 2);
  valu_row<1>(b, "v_exp_f32 (+ v_sub)", 1);
  valu_row<1>(b, "v_exp_f32 (+ v_sub)", 2);
  valu_row<2>(b, "degree-3 polynomial exp2 (+ v_sub)", 1);
  valu_row<2>(b, "degree-3 polynomial exp2 (+ v_sub)", 2);

  printf("\n## One wavefront per SIMD: its MFMAs with its own VALU work\n\n");
  printf("| FMAs per MFMA | exps per MFMA | cycles per step (one 32x32x16 MFMA = 32 cycles alone) |\n|---|---|---|\n");
  overlap_row<0, 0>(b);
  overlap_row<2, 0>(b);
  overlap_row<4, 0>(b);
  overlap_row<6, 0>(b);
  overlap_row<8, 0>(b);
  overlap_row<0, 1>(b);
  overlap_row<0, 2>(b);
  overlap_row<4, 1>(b);

  printf("\n## LDS reads (16 in flight per wavefront)\n\n");
  printf("| read | waves per CU | bytes/clk per CU |\n|---|---|---|\n");
  lds_row<0>(b, "ds_read_b128, swizzled rows", 4);
  lds_row<0>(b, "ds_read_b128, swizzled rows", 8);
  lds_row<0>(b, "ds_read_b128, swizzled rows", 16);
  lds_row<1>(b, "ds_read_b128, one column of 32 rows", 4);
  lds_row<1>(b, "ds_read_b128, one column of 32 rows", 16);
  lds_row<2>(b, "ds_read_b64_tr_b16, swizzled rows", 4);
  lds_row<2>(b, "ds_read_b64_tr_b16, swizzled rows", 8);
  lds_row<2>(b, "ds_read_b64_tr_b16, swizzled rows", 16);

  atomic_section();

  UB_CHECK(hipFree(b.in));
  UB_CHECK(hipFree(b.out));
  UB_CHECK(hipFree(b.cyc));
  return 0;
}

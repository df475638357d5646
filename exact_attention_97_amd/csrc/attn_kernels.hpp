// attn_kernels.hpp - host-side launch interface between the C ABI layer and
// the kernel translation units.  Plain structs of device pointers and sizes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn97 {

// Kernel exp2 modes of the forward kernels: native v_exp_f32, the polynomial
// on the FMA pipe, or mixed with the polynomial taking q of every four
// elements (q = 1, 2, 3: a quarter, half, three quarters).
constexpr int kExpNative = 0, kExpPoly = 1;
constexpr int exp_mix(int q) { return 1 + q; }  // q = 1..3 -> 2..4

struct FwdArgs {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  float* LSE;
  int B, H, S, D;
  int causal;
  int exp_mode;    // kernel exp2 mode (kExpNative, kExpPoly, exp_mix(q))
  float C;         // |scale| * log2(e)
  uint32_t qsign;  // 0x80008000 flips the sign of Q (negative scale), else 0
  float tau;       // conditional rescale threshold, log2 units
};

struct BwdArgs {
  const void* Q;
  const void* K;
  const void* V;
  const void* O;
  const void* dO;
  const float* LSE;
  void* dQ;
  void* dK;
  void* dV;
  float* delta;  // workspace: fp32 [B,H,S], Delta_i = sum_d dO_id O_id
  float* nlse2;  // workspace: fp32 [B,H,S], -LSE_i * log2(e)
  float* dq32;   // workspace: fp32 [B,H,S,D] (atomic mode)
  int B, H, S, D;
  int causal;
  float scale;
};

// Workspace layout of attn_bwd: delta and nlse2 (each rounded up to 256
// bytes), then dq32 in atomic mode.
inline size_t bwd_delta_bytes(int B, int H, int S) {
  size_t n = (size_t)B * H * S * sizeof(float);
  return (n + 255) & ~(size_t)255;
}
inline size_t bwd_dq32_bytes(int B, int H, int S, int D) {
  return (size_t)B * H * S * D * sizeof(float);
}

// Split-KV forward: per-split partial results in the workspace, then a merge.
struct SplitKvLaunch {
  int Sk;        // keys (the queries are FwdArgs::S)
  int nsplit;    // number of key chunks
  int kchunk;    // keys per chunk, a multiple of fwd_tile_keys(D)
  float* Opart;  // [nsplit, B*H, S, D] fp32
  float* Lpart;  // [nsplit, B*H, S] fp32
};

// FP8 forward: the quantized operands and their scales in one caller-owned
// buffer (regions in this order, each rounded up to 256 bytes); Sp is S
// rounded up to 128, rows past S are zero.
struct Fp8Buf {
  int Sp;
  uint8_t* q8;   // [B*H, Sp, 128] E4M3, transformed Q
  uint8_t* k8;   // [B*H, Sp, 128] E4M3, transformed K
  uint8_t* v8t;  // [B*H, 128, Sp] E4M3, V transposed, keys permuted in 64-groups
  float* qs;     // [B*H, Sp] per-row Q scales
  float* ks;     // [B*H] per-head K scales
  float* vs;     // [B*H, 128] per-column V scales
  float* vpart;  // scratch: V's column maxima, [B*H, 128] float
  void* kmax;    // scratch: K's head maxima (of the transformed rows), [B*H] double
  size_t offsets[7];
};
// Byte size of the buffer; fills *f from `base` when f is not null.
size_t fp8_layout(int B, int H, int S, int D, void* base, Fp8Buf* f);
hipError_t launch_fp8_quantize(const void* Q, const void* K, const void* V, const float* signs, const Fp8Buf& f,
                               int B, int H, int S, hipStream_t st);
hipError_t launch_fp8_dot_eval(const void* A, const void* Bt, float* C, long nblk, hipStream_t st);
hipError_t launch_fwd_fp8(const Fp8Buf& f, void* O, float* LSE, int B, int H, int S, float C, uint32_t qsign,
                          float tau, int causal, hipStream_t st);

// Kernel names used by the timing hooks.
enum KernelId {
  KID_FWD = 0,
  KID_BWD_PRE,
  KID_BWD_MAIN,
  KID_DQ_CONVERT,
  KID_BWD_DKDV,
  KID_BWD_DQ,
  KID_FWD_SPLITKV,
  KID_SPLITKV_MERGE,
  KID_FP8_QUANT,
  KID_FWD_FP8,
  KID_COUNT
};

// Kernel variants kept for measurement (0 = the default kernel).  The
// choice comes from attn_set_variant, else from the environment variables
// ATTN97_FWD_VARIANT, ATTN97_DQ_VARIANT, ATTN97_DKDV_VARIANT (read once).
enum VariantSlot { VAR_FWD = 0, VAR_DQ, VAR_DKDV, VAR_COUNT };
int kernel_variant(int slot);

// Called by the launchers around each kernel launch (no-ops unless timing is on).
void prof_begin(int kid, hipStream_t st);
void prof_end(int kid, hipStream_t st);

hipError_t launch_fwd(const FwdArgs& a, hipStream_t st);
hipError_t launch_fwd_splitkv(const FwdArgs& a, const SplitKvLaunch& p, hipStream_t st);
int fwd_tile_keys(int D);     // keys per tile of the forward kernel for head dim D
int fwd_tile_queries(int D);  // queries per workgroup of the forward kernel
hipError_t launch_exp2_eval(const float* x, float* y, long n, int mode, hipStream_t st);
hipError_t launch_bwd_atomic(const BwdArgs& a, hipStream_t st);
hipError_t launch_bwd_split(const BwdArgs& a, hipStream_t st);
hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t st);
bool bwd_supported(int D, bool atomic);

}  // namespace attn97

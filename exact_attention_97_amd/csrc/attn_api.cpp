// attn_api.cpp - the C ABI declared in include/attn97.h: argument checks,
// option handling, workspace layout, kernel dispatch and the timing hooks.
// Nothing here allocates device memory or synchronises with the device
// (except attn_prof_collect, which waits on its own timing events).
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdlib.h>
#include <stdint.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "attn97.h"
#include "attn_kernels.hpp"

namespace {

constexpr float kLog2eHost = 1.4426950408889634f;

bool misaligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; }

attn_status check_shape(int B, int H, int S, int D) {
  if (B < 1 || H < 1 || S < 1) return ATTN_ERR_SHAPE;
  if (D != 64 && D != 128 && D != 256) return ATTN_ERR_UNSUPPORTED;
  const double elems = (double)B * H * S * D;
  if (elems > 2147483647.0) return ATTN_ERR_SHAPE;
  return ATTN_OK;
}

// Largest accepted rescale threshold (log2 units).  An unnormalised
// probability is at most 2^tau and a row sums at most S of them, so with
// tau <= 64 the fp32 row sum and accumulators stay below 2^64 * 2^31 * |v|,
// far from fp32 overflow (2^128), for every supported length.
constexpr float kMaxTau = 64.0f;
// The FP8 forward rounds unnormalised probabilities (at most 2^tau) to E4M3,
// whose largest value is 448.
constexpr float kMaxTauFp8 = 8.0f;

attn_status read_opts(const attn_opts* in, attn_opts* out) {
  attn_default_opts(out);
  if (in == nullptr) return ATTN_OK;
  if (in->exp_mode < 0 || in->exp_mode > 2) return ATTN_ERR_UNSUPPORTED;
  if (in->bwd_mode < 0 || in->bwd_mode > 1) return ATTN_ERR_UNSUPPORTED;
  if (!(in->rescale_tau >= 0.0f && in->rescale_tau <= kMaxTau)) return ATTN_ERR_VALUE;
  if (!(in->poly_fraction >= 0.0f && in->poly_fraction <= 1.0f)) return ATTN_ERR_VALUE;
  *out = *in;
  return ATTN_OK;
}

// Kernel exp2 mode of validated options: the mixed mode's fraction is
// rounded to the nearest quarter (ties to even); a fraction that rounds to 0
// or 1 runs the native or the polynomial kernel.
int kernel_exp_mode(const attn_opts& o) {
  if (o.exp_mode == ATTN_EXP_NATIVE) return attn97::kExpNative;
  if (o.exp_mode == ATTN_EXP_POLY) return attn97::kExpPoly;
  const long q = lrintf(o.poly_fraction * 4.0f);
  if (q <= 0) return attn97::kExpNative;
  if (q >= 4) return attn97::kExpPoly;
  return attn97::exp_mix((int)q);
}

// ---- timing hooks -----------------------------------------------------------
struct ProfRec {
  int kid;
  hipEvent_t start, stop;
};
constexpr size_t kMaxProf = 65536;
bool g_prof_on = false;
std::vector<ProfRec> g_prof_pool;  // events, created on first use and reused
size_t g_prof_used = 0;
size_t g_prof_open = (size_t)-1;

// kernel variant overrides (-1: not set, use the environment)
int g_variant[attn97::VAR_COUNT] = {-1, -1, -1};
int g_variant_env[attn97::VAR_COUNT] = {-1, -1, -1};

}  // namespace

namespace attn97 {

int kernel_variant(int slot) {
  if (slot < 0 || slot >= VAR_COUNT) return 0;
  if (g_variant[slot] >= 0) return g_variant[slot];
  if (g_variant_env[slot] < 0) {
    static const char* names[VAR_COUNT] = {"ATTN97_FWD_VARIANT", "ATTN97_DQ_VARIANT", "ATTN97_DKDV_VARIANT"};
    const char* e = getenv(names[slot]);
    const int v = e ? atoi(e) : 0;
    g_variant_env[slot] = v < 0 ? 0 : v;
  }
  return g_variant_env[slot];
}

void prof_begin(int kid, hipStream_t st) {
  g_prof_open = (size_t)-1;
  if (!g_prof_on || g_prof_used >= kMaxProf) return;
  if (g_prof_used == g_prof_pool.size()) {
    ProfRec r{kid, nullptr, nullptr};
    if (hipEventCreate(&r.start) != hipSuccess) return;
    if (hipEventCreate(&r.stop) != hipSuccess) {
      (void)hipEventDestroy(r.start);
      return;
    }
    g_prof_pool.push_back(r);
  }
  ProfRec& r = g_prof_pool[g_prof_used];
  r.kid = kid;
  if (hipEventRecord(r.start, st) != hipSuccess) return;
  g_prof_open = g_prof_used;
}

void prof_end(int kid, hipStream_t st) {
  if (g_prof_open == (size_t)-1) return;
  ProfRec& r = g_prof_pool[g_prof_open];
  g_prof_open = (size_t)-1;
  if (r.kid != kid) return;
  if (hipEventRecord(r.stop, st) != hipSuccess) return;
  ++g_prof_used;
}

}  // namespace attn97

extern "C" {

void attn_default_opts(attn_opts* opts) {
  if (opts == nullptr) return;
  opts->exp_mode = ATTN_EXP_NATIVE;
  opts->poly_fraction = 0.5f;
  opts->rescale_tau = 8.0f;
  opts->bwd_mode = ATTN_BWD_SPLIT;
}

const char* attn_version(void) { return "attn97 0.1.0 (gfx950)"; }

const char* attn_strerror(attn_status s) {
  switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "invalid shape (B, H and S must be >= 1; tensors below 2^31 elements)";
    case ATTN_ERR_UNSUPPORTED: return "unsupported head dimension or option";
    case ATTN_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case ATTN_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case ATTN_ERR_HIP: return "HIP runtime error at launch";
    case ATTN_ERR_VALUE: return "scale or an option value is not finite or out of range";
    case ATTN_ERR_SCRATCH_LIMIT:
      return "the shape needs more workspace than the fixed scratch of attn_bwd_noalloc (ATTN_NOALLOC_SCRATCH_BYTES)";
  }
  return "unknown status";
}

attn_status attn_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H,
                     int S, int D, float scale, int causal, const attn_opts* opts, void* stream) {
  if (!Q || !K || !V || !O || !LSE) return ATTN_ERR_NULL;
  attn_status st = check_shape(B, H, S, D);
  if (st != ATTN_OK) return st;
  if (misaligned(Q, 16) || misaligned(K, 16) || misaligned(V, 16) || misaligned(O, 16) ||
      misaligned(LSE, 16))
    return ATTN_ERR_ALIGN;
  if (!isfinite(scale)) return ATTN_ERR_VALUE;
  attn_opts o;
  st = read_opts(opts, &o);
  if (st != ATTN_OK) return st;

  attn97::FwdArgs a;
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.O = O;
  a.LSE = LSE;
  a.B = B;
  a.H = H;
  a.S = S;
  a.D = D;
  a.causal = causal ? 1 : 0;
  a.exp_mode = kernel_exp_mode(o);
  a.C = fabsf(scale) * kLog2eHost;
  a.qsign = (scale < 0.0f) ? 0x80008000u : 0u;
  a.tau = o.rescale_tau;
  hipError_t e = attn97::launch_fwd(a, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // extern "C"

namespace {

size_t round256(size_t n) { return (n + 255) & ~(size_t)255; }

// Validated shape of a split-KV call and its split plan (shared by the
// workspace query and the call, so both always agree).
struct SplitPlan {
  int nsplit = 0, kchunk = 0;
  size_t opart_bytes = 0, lpart_bytes = 0;
};

attn_status plan_splitkv(int B, int H, int Sq, int Sk, int D, int causal, int num_splits, SplitPlan* p) {
  if (B < 1 || H < 1 || Sq < 1 || Sk < 1) return ATTN_ERR_SHAPE;
  if (D != 64 && D != 128 && D != 256) return ATTN_ERR_UNSUPPORTED;
  if ((double)B * H * Sq * D > 2147483647.0 || (double)B * H * Sk * D > 2147483647.0) return ATTN_ERR_SHAPE;
  if (causal && Sk < Sq) return ATTN_ERR_SHAPE;  // the queries are the last Sq of the Sk positions
  if (num_splits < 0) return ATTN_ERR_VALUE;
  const int bc = attn97::fwd_tile_keys(D), br = attn97::fwd_tile_queries(D);
  const long ntiles = (Sk + bc - 1) / bc;
  long ns = num_splits;
  if (ns == 0) {  // enough workgroups for two per compute unit
    const long wgs = (long)((Sq + br - 1) / br) * B * H;
    ns = (512 + wgs - 1) / wgs;
  }
  ns = ns < 1 ? 1 : (ns > ntiles ? ntiles : ns);
  const long tiles_per = (ntiles + ns - 1) / ns;
  p->kchunk = (int)(tiles_per * bc);
  p->nsplit = (int)((Sk + p->kchunk - 1) / p->kchunk);
  const double parts = (double)p->nsplit * B * H * Sq;
  if (parts * D > 9.0e15) return ATTN_ERR_SHAPE;
  p->opart_bytes = round256((size_t)p->nsplit * B * H * Sq * D * sizeof(float));
  p->lpart_bytes = round256((size_t)p->nsplit * B * H * Sq * sizeof(float));
  return ATTN_OK;
}

}  // namespace

extern "C" {

size_t attn_fwd_splitkv_workspace_bytes(int B, int H, int Sq, int Sk, int D, int causal, int num_splits) {
  SplitPlan p;
  if (plan_splitkv(B, H, Sq, Sk, D, causal, num_splits, &p) != ATTN_OK) return 0;
  return p.opart_bytes + p.lpart_bytes;
}

attn_status attn_fwd_splitkv(const void* Q, const void* K, const void* V, void* O, float* LSE, void* workspace,
                             size_t workspace_bytes, int B, int H, int Sq, int Sk, int D, float scale, int causal,
                             int num_splits, const attn_opts* opts, void* stream) {
  if (!Q || !K || !V || !O || !LSE) return ATTN_ERR_NULL;
  SplitPlan p;
  attn_status st = plan_splitkv(B, H, Sq, Sk, D, causal ? 1 : 0, num_splits, &p);
  if (st != ATTN_OK) return st;
  if (misaligned(Q, 16) || misaligned(K, 16) || misaligned(V, 16) || misaligned(O, 16) || misaligned(LSE, 16))
    return ATTN_ERR_ALIGN;
  if (!isfinite(scale)) return ATTN_ERR_VALUE;
  attn_opts o;
  st = read_opts(opts, &o);
  if (st != ATTN_OK) return st;
  if (workspace == nullptr || workspace_bytes < p.opart_bytes + p.lpart_bytes || misaligned(workspace, 256))
    return ATTN_ERR_WORKSPACE;

  attn97::FwdArgs a;
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.O = O;
  a.LSE = LSE;
  a.B = B;
  a.H = H;
  a.S = Sq;
  a.D = D;
  a.causal = causal ? 1 : 0;
  a.exp_mode = kernel_exp_mode(o);
  a.C = fabsf(scale) * kLog2eHost;
  a.qsign = (scale < 0.0f) ? 0x80008000u : 0u;
  a.tau = o.rescale_tau;
  attn97::SplitKvLaunch l;
  l.Sk = Sk;
  l.nsplit = p.nsplit;
  l.kchunk = p.kchunk;
  l.Opart = static_cast<float*>(workspace);
  l.Lpart = reinterpret_cast<float*>(static_cast<char*>(workspace) + p.opart_bytes);
  hipError_t e = attn97::launch_fwd_splitkv(a, l, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

size_t attn_bwd_workspace_bytes(int B, int H, int S, int D, int causal, const attn_opts* opts) {
  (void)causal;
  if (check_shape(B, H, S, D) != ATTN_OK) return 0;
  attn_opts o;
  if (read_opts(opts, &o) != ATTN_OK) return 0;
  size_t n = 2 * attn97::bwd_delta_bytes(B, H, S);
  if (o.bwd_mode == ATTN_BWD_ATOMIC) n += attn97::bwd_dq32_bytes(B, H, S, D);
  return n;
}

}  // extern "C"

namespace {

// Argument checks of attn_bwd and attn_bwd_noalloc (everything but the
// workspace); fills the options and the workspace size the call needs.
attn_status check_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* LSE,
                      void* dQ, void* dK, void* dV, int B, int H, int S, int D, float scale, int causal,
                      const attn_opts* opts, attn_opts* o, size_t* need) {
  if (!Q || !K || !V || !O || !dO || !LSE || !dQ || !dK || !dV) return ATTN_ERR_NULL;
  attn_status st = check_shape(B, H, S, D);
  if (st != ATTN_OK) return st;
  if (misaligned(Q, 16) || misaligned(K, 16) || misaligned(V, 16) || misaligned(O, 16) ||
      misaligned(dO, 16) || misaligned(LSE, 16) || misaligned(dQ, 16) || misaligned(dK, 16) ||
      misaligned(dV, 16))
    return ATTN_ERR_ALIGN;
  if (!isfinite(scale)) return ATTN_ERR_VALUE;
  st = read_opts(opts, o);
  if (st != ATTN_OK) return st;
  if (!attn97::bwd_supported(D, o->bwd_mode == ATTN_BWD_ATOMIC)) return ATTN_ERR_UNSUPPORTED;
  *need = attn_bwd_workspace_bytes(B, H, S, D, causal, o);
  return ATTN_OK;
}

// The backward launches on a checked, large enough workspace.
attn_status run_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* LSE,
                    void* dQ, void* dK, void* dV, void* workspace, int B, int H, int S, int D, float scale,
                    int causal, const attn_opts& o, void* stream) {
  attn97::BwdArgs a;
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.O = O;
  a.dO = dO;
  a.LSE = LSE;
  a.dQ = dQ;
  a.dK = dK;
  a.dV = dV;
  const size_t vec_bytes = attn97::bwd_delta_bytes(B, H, S);
  a.delta = static_cast<float*>(workspace);
  a.nlse2 = reinterpret_cast<float*>(static_cast<char*>(workspace) + vec_bytes);
  a.dq32 = (o.bwd_mode == ATTN_BWD_ATOMIC) ? reinterpret_cast<float*>(static_cast<char*>(workspace) + 2 * vec_bytes)
                                          : nullptr;
  a.B = B;
  a.H = H;
  a.S = S;
  a.D = D;
  a.causal = causal ? 1 : 0;
  a.scale = scale;
  hipError_t e = (o.bwd_mode == ATTN_BWD_ATOMIC) ? attn97::launch_bwd_atomic(a, (hipStream_t)stream)
                                                 : attn97::launch_bwd_split(a, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

// ---- the no-allocation entry point's scratch ------------------------------
// A fixed device array in the library's code object: every GPU the library
// runs on holds its own copy, at its own address, until the process ends.
// In host code `scratch` is only a stand-in for the symbol: its device
// address comes from hipGetSymbolAddress, once per device (with that device
// current), and only that address is passed to kernels.
static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// The current device's scratch address (looked up on the first call there).
attn_status current_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_ERR_HIP;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = p;
  });
  if (g_scratch_err[dev] != hipSuccess || g_scratch_ptr[dev] == nullptr) return ATTN_ERR_HIP;
  *out = g_scratch_ptr[dev];
  return ATTN_OK;
}

}  // namespace

extern "C" {

attn_status attn_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                     const float* LSE, void* dQ, void* dK, void* dV, void* workspace,
                     size_t workspace_bytes, int B, int H, int S, int D, float scale, int causal,
                     const attn_opts* opts, void* stream) {
  attn_opts o;
  size_t need = 0;
  attn_status st = check_bwd(Q, K, V, O, dO, LSE, dQ, dK, dV, B, H, S, D, scale, causal, opts, &o, &need);
  if (st != ATTN_OK) return st;
  if (workspace == nullptr || workspace_bytes < need || misaligned(workspace, 256))
    return ATTN_ERR_WORKSPACE;
  return run_bwd(Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, B, H, S, D, scale, causal, o, stream);
}

attn_status attn_bwd_noalloc(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                             const float* LSE, void* dQ, void* dK, void* dV, int B, int H, int S, int D,
                             float scale, int causal, const attn_opts* opts, void* stream) {
  attn_opts o;
  size_t need = 0;
  attn_status st = check_bwd(Q, K, V, O, dO, LSE, dQ, dK, dV, B, H, S, D, scale, causal, opts, &o, &need);
  if (st != ATTN_OK) return st;
  if (need > (size_t)ATTN_NOALLOC_SCRATCH_BYTES) return ATTN_ERR_SCRATCH_LIMIT;
  void* ws = nullptr;
  st = current_scratch(&ws);
  if (st != ATTN_OK) return st;
  // every byte the kernels read from the scratch is written first in this
  // call (Delta and -LSE log2e by the preprocessing kernel, which also zeroes
  // the dQ accumulator in the atomic mode), so what an earlier call left
  // there does not matter
  return run_bwd(Q, K, V, O, dO, LSE, dQ, dK, dV, ws, B, H, S, D, scale, causal, o, stream);
}

size_t attn_fp8_buffer_bytes(int B, int H, int S, int D) {
  if (check_shape(B, H, S, D) != ATTN_OK || D != 128) return 0;
  return attn97::fp8_layout(B, H, S, D, nullptr, nullptr);
}

attn_status attn_fp8_buffer_offsets(int B, int H, int S, int D, size_t offsets[7]) {
  if (!offsets) return ATTN_ERR_NULL;
  attn_status st = check_shape(B, H, S, D);
  if (st != ATTN_OK) return st;
  if (D != 128) return ATTN_ERR_UNSUPPORTED;
  attn97::Fp8Buf f;
  attn97::fp8_layout(B, H, S, D, nullptr, &f);
  for (int i = 0; i < 7; ++i) offsets[i] = f.offsets[i];
  return ATTN_OK;
}

attn_status attn_fp8_quantize(const void* Q, const void* K, const void* V, const float* signs, void* buf,
                              size_t buf_bytes, int B, int H, int S, int D, void* stream) {
  if (!Q || !K || !V) return ATTN_ERR_NULL;
  attn_status st = check_shape(B, H, S, D);
  if (st != ATTN_OK) return st;
  if (D != 128) return ATTN_ERR_UNSUPPORTED;
  if (misaligned(Q, 16) || misaligned(K, 16) || misaligned(V, 16) || misaligned(signs, 4)) return ATTN_ERR_ALIGN;
  attn97::Fp8Buf f;
  const size_t need = attn97::fp8_layout(B, H, S, D, buf, &f);
  if (buf == nullptr || buf_bytes < need || misaligned(buf, 256)) return ATTN_ERR_WORKSPACE;
  hipError_t e = attn97::launch_fp8_quantize(Q, K, V, signs, f, B, H, S, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

attn_status attn_fwd_fp8(const void* buf, size_t buf_bytes, void* O, float* LSE, int B, int H, int S, int D,
                         float scale, int causal, const attn_opts* opts, void* stream) {
  if (!O || !LSE) return ATTN_ERR_NULL;
  attn_status st = check_shape(B, H, S, D);
  if (st != ATTN_OK) return st;
  if (D != 128) return ATTN_ERR_UNSUPPORTED;
  if (misaligned(O, 16) || misaligned(LSE, 16)) return ATTN_ERR_ALIGN;
  if (!isfinite(scale)) return ATTN_ERR_VALUE;
  attn_opts o;
  st = read_opts(opts, &o);
  if (st != ATTN_OK) return st;
  attn97::Fp8Buf f;
  const size_t need = attn97::fp8_layout(B, H, S, D, const_cast<void*>(buf), &f);
  if (buf == nullptr || buf_bytes < need || misaligned(buf, 256)) return ATTN_ERR_WORKSPACE;
  // P is stored in E4M3, whose largest finite value is 448; unnormalised
  // probabilities stay below 2^tau, so the FP8 kernel applies tau <= 8
  // (2^8 = 256 < 448) whatever larger value the options give.
  const float tau = o.rescale_tau < kMaxTauFp8 ? o.rescale_tau : kMaxTauFp8;
  hipError_t e = attn97::launch_fwd_fp8(f, O, LSE, B, H, S, fabsf(scale) * kLog2eHost,
                                        (scale < 0.0f) ? 0x80808080u : 0u, tau, causal ? 1 : 0, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

attn_status attn_fp8_dot_eval(const void* A, const void* Bt, float* C, long nblk, void* stream) {
  if (nblk < 0) return ATTN_ERR_SHAPE;
  if (nblk == 0) return ATTN_OK;
  if (!A || !Bt || !C) return ATTN_ERR_NULL;
  if (misaligned(A, 16) || misaligned(Bt, 16) || misaligned(C, 16)) return ATTN_ERR_ALIGN;
  if ((double)nblk * 32 * 128 > 9.0e15) return ATTN_ERR_SHAPE;
  hipError_t e = attn97::launch_fp8_dot_eval(A, Bt, C, nblk, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

attn_status attn_exp2_eval(const float* x, float* y, long n, int mode, void* stream) {
  if (n < 0) return ATTN_ERR_SHAPE;
  if (mode != ATTN_EXP_NATIVE && mode != ATTN_EXP_POLY) return ATTN_ERR_UNSUPPORTED;
  if (n == 0) return ATTN_OK;
  if (!x || !y) return ATTN_ERR_NULL;
  if (misaligned(x, 4) || misaligned(y, 4)) return ATTN_ERR_ALIGN;
  hipError_t e = attn97::launch_exp2_eval(x, y, n, mode, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

attn_status attn_set_variant(const char* kernel, int variant) {
  if (!kernel) return ATTN_ERR_NULL;
  static const char* names[attn97::VAR_COUNT] = {"fwd", "bwd_dq", "bwd_dkdv"};
  static const int count[attn97::VAR_COUNT] = {3, 3, 2};  // variants 0 .. count-1
  for (int i = 0; i < attn97::VAR_COUNT; ++i) {
    if (strcmp(kernel, names[i]) != 0) continue;
    if (variant < -1 || variant >= count[i]) return ATTN_ERR_VALUE;
    g_variant[i] = variant;
    return ATTN_OK;
  }
  return ATTN_ERR_UNSUPPORTED;
}

attn_status attn_prof_enable(int on) {
  g_prof_on = on != 0;
  return ATTN_OK;
}

attn_status attn_prof_reset(void) {
  g_prof_used = 0;
  g_prof_open = (size_t)-1;
  return ATTN_OK;
}

attn_status attn_prof_collect(const char* kernel, int* count, double* total_ms) {
  if (!kernel || !count || !total_ms) return ATTN_ERR_NULL;
  static const char* names[attn97::KID_COUNT] = {"fwd",         "bwd_pre",       "bwd_main",     "dq_convert",
                                                "bwd_dkdv",    "bwd_dq",        "fwd_splitkv", "splitkv_merge",
                                                "fp8_quantize", "fwd_fp8"};
  int kid = -1;
  for (int i = 0; i < attn97::KID_COUNT; ++i)
    if (strcmp(kernel, names[i]) == 0) kid = i;
  if (kid < 0) return ATTN_ERR_UNSUPPORTED;
  int n = 0;
  double ms = 0.0;
  for (size_t i = 0; i < g_prof_used; ++i) {
    ProfRec& r = g_prof_pool[i];
    if (r.kid != kid) continue;
    if (hipEventSynchronize(r.stop) != hipSuccess) return ATTN_ERR_HIP;
    float t = 0.0f;
    if (hipEventElapsedTime(&t, r.start, r.stop) != hipSuccess) return ATTN_ERR_HIP;
    ms += t;
    ++n;
  }
  *count = n;
  *total_ms = ms;
  return ATTN_OK;
}

}  // extern "C"

/*
 * attn97.h - C ABI of the exact fused attention library for AMD MI355X (gfx950).
 *
 * The library computes exact scaled-dot-product attention
 *     O = softmax(scale * Q K^T) V
 * for one GPU.  Attention is two matrix products with a softmax between
 * them: the scores S = Q K^T and the output O = P V (page "FlashAttention-4 :
 * comment Together AI a accéléré l'attention sur GPU Blackwell", section
 * "Pourquoi l'approche standard ne fonctionne plus"; page "FlashAttention-3 и
 * FlashAttention-4", section "Режим 2-CTA MMA", which also names the
 * softmax, normalisation, masking and row reductions between the products).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Q, K, V, O, dO, dQ, dK, dV are bfloat16 tensors in contiguous row-major
 *    layout [B, H, S, D] (D fastest), resident in device memory.
 *  - LSE is float32 [B, H, S]: the natural-log log-sum-exp of each row of
 *    scaled scores, LSE_i = ln sum_j exp(scale * q_i . k_j) over visible j.
 *  - causal != 0 hides key j from query i when j > i (0-based indices).
 *    Queries and keys have the same length S, so no row is fully hidden.
 *  - Every pointer is a device pointer, owned by the caller, and must be
 *    16-byte aligned.  Inputs are read-only.  Outputs must not alias inputs.
 *  - B, H, S >= 1 and D in {64, 128, 256}; S need not be a multiple of any
 *    tile size.  B*H*S*D must fit in 2^31 - 1 elements per tensor.
 *  - scale must be finite (any sign; 0 gives the mean of the visible rows).
 *  - stream is a hipStream_t (NULL = the default stream).  Calls are
 *    asynchronous with respect to the host; the library never synchronises
 *    and never allocates device memory.  Its only state is process-global
 *    diagnostics (attn_set_variant, the timing hooks attn_prof_*); with those
 *    left alone, calls on different streams and threads may run concurrently.
 *  - Errors are return codes only.  Argument errors are detected before
 *    anything is launched.  A failed launch returns ATTN_ERR_HIP; a fault
 *    inside a kernel surfaces at the caller's next synchronisation.
 */
#ifndef ATTN97_H
#define ATTN97_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_NULL = 1,        /* a required pointer is NULL                 */
    ATTN_ERR_SHAPE = 2,       /* B, H or S < 1, or a tensor too large       */
    ATTN_ERR_UNSUPPORTED = 3, /* D not in {64,128,256}, or an unknown option */
    ATTN_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned            */
    ATTN_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required     */
    ATTN_ERR_HIP = 6,         /* the HIP runtime rejected a launch           */
    ATTN_ERR_VALUE = 7,       /* scale or an option value is not finite / out of range */
    ATTN_ERR_SCRATCH_LIMIT = 8 /* attn_bwd_noalloc: the shape needs more than its fixed scratch */
} attn_status;

/* How the forward kernel computes exp2 of the shifted scores.  The pages
 * describe computing the softmax exponential in software with a polynomial
 * on the fused multiply-add units instead of the special-function units
 * (page "FlashAttention-3 и FlashAttention-4", section "Программная эмуляция
 * экспоненты"; abstract of "FlashAttention-4: Algorithm and Kernel Pipelining
 * Co-Design for Asymmetric Hardware Scaling"). */
typedef enum {
    ATTN_EXP_NATIVE = 0, /* hardware v_exp_f32 for every element                           */
    ATTN_EXP_POLY = 1,   /* range reduction + degree-3 polynomial on the FMA pipe           */
    ATTN_EXP_MIXED = 2   /* a fraction poly_fraction of the scores polynomial, the rest native */
} attn_exp_mode;

/* How the backward pass forms dQ.  The pages name the atomic additions of
 * the backward pass as an overhead at long sequence lengths (page
 * "FlashAttention-3 и FlashAttention-4", section "Режим 2-CTA MMA"). */
typedef enum {
    ATTN_BWD_ATOMIC = 0, /* one kernel per key tile; dQ summed with fp32 atomics into the workspace
                            (D = 64 and 128 only; D = 256 returns ATTN_ERR_UNSUPPORTED)            */
    ATTN_BWD_SPLIT = 1   /* a dK/dV kernel plus a separate dQ kernel; no atomics, deterministic    */
} attn_bwd_mode;

typedef struct {
    int exp_mode;        /* attn_exp_mode; default ATTN_EXP_NATIVE                              */
    float poly_fraction; /* ATTN_EXP_MIXED only: share of each lane's scores whose exp2 takes the
                            polynomial, in [0, 1], rounded to the nearest quarter (ties to even);
                            0 runs the native kernel and 1 the polynomial one.  The software
                            exponential covers only part of the exponentials (page
                            "FlashAttention-3 и FlashAttention-4", section "Программная эмуляция
                            экспоненты").  Default 0.5.  Outside [0, 1] or NaN: ATTN_ERR_VALUE. */
    float rescale_tau;   /* conditional rescaling threshold in log2 units, in [0, 64]; default 8.
                            The running row maximum used to shift the scores is only moved when
                            some score of a wavefront's rows could exceed it by more than tau, so
                            unnormalised probabilities stay at most 2^tau.  0 = always rescale.
                            (Conditional softmax rescaling: abstract of "FlashAttention-4:
                            Algorithm and Kernel Pipelining Co-Design for Asymmetric Hardware
                            Scaling".)  The result is the same for every tau up to rounding.
                            Above 64 (where 2^tau times S probabilities could approach the fp32
                            range), negative or NaN: ATTN_ERR_VALUE.                          */
    int bwd_mode;        /* attn_bwd_mode; default ATTN_BWD_SPLIT                               */
} attn_opts;

/* Defaults: {ATTN_EXP_NATIVE, 0.5f, 8.0f, ATTN_BWD_SPLIT}. */
void attn_default_opts(attn_opts* opts);

/*
 * Forward pass.
 *   in : Q, K, V   bf16 [B,H,S,D]
 *   out: O         bf16 [B,H,S,D]  O = softmax(scale*Q K^T (+ causal mask)) V,
 *                                  rounded to nearest even from fp32
 *        LSE       fp32 [B,H,S]    natural-log log-sum-exp of each row
 *   opts may be NULL (defaults).
 */
attn_status attn_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE,
                     int B, int H, int S, int D, float scale, int causal,
                     const attn_opts* opts, void* stream);

/*
 * Bytes of device workspace attn_bwd needs for this shape and mode: two
 * per-row fp32 vectors [B,H,S] (Delta_i = sum_d dO_id * O_id, and
 * -LSE_i * log2(e)), each padded to a multiple of 256 bytes, and, in
 * ATTN_BWD_ATOMIC mode, the fp32 dQ accumulator [B,H,S,D].  Returns 0 for
 * invalid shapes.
 */
size_t attn_bwd_workspace_bytes(int B, int H, int S, int D, int causal, const attn_opts* opts);

/*
 * Backward pass.  P is recomputed from LSE (it is never stored):
 *   P = exp(scale*Q K^T - LSE), dV = P^T dO, dP = dO V^T,
 *   dS = P * (dP - Delta), dQ = scale * dS K, dK = scale * dS^T Q.
 *   in : Q, K, V, O, dO  bf16 [B,H,S,D];  LSE fp32 [B,H,S] from attn_fwd with
 *        the same scale and causal flag
 *   out: dQ, dK, dV      bf16 [B,H,S,D]
 *   workspace: caller-owned device memory of at least
 *        attn_bwd_workspace_bytes(...) bytes, 256-byte aligned; its contents
 *        on entry do not matter and are overwritten.  Two calls in flight at
 *        once must not share a workspace.
 *   D = 256 runs in ATTN_BWD_SPLIT mode only (two workgroups per key tile,
 *   each forming half of the dK / dV columns); ATTN_BWD_ATOMIC returns
 *   ATTN_ERR_UNSUPPORTED there.
 */
attn_status attn_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                     const float* LSE, void* dQ, void* dK, void* dV,
                     void* workspace, size_t workspace_bytes,
                     int B, int H, int S, int D, float scale, int causal,
                     const attn_opts* opts, void* stream);

/*
 * Backward pass that allocates nothing, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): attn_bwd with its workspace taken from a
 * fixed device array inside the library, ATTN_NOALLOC_SCRATCH_BYTES per GPU,
 * held by every GPU the library runs on until the process ends.  The caller
 * still passes inputs and outputs.  Arguments and results as attn_bwd.
 *   The scratch of the current device is used (its address is looked up once
 *   per device, on the first call there); the stream must belong to that
 *   device.  Shapes whose attn_bwd_workspace_bytes(...) exceed
 *   ATTN_NOALLOC_SCRATCH_BYTES return ATTN_ERR_SCRATCH_LIMIT before anything
 *   is launched: in the split mode (default) up to 4 194 240 rows B*H*S, in
 *   the atomic mode far fewer (its fp32 dQ accumulator is B*H*S*D floats).
 *   All calls on one GPU share its scratch and each leaves its contents
 *   behind: calls that overlap on one GPU (other streams, other threads)
 *   race and must not be issued; calls ordered on one stream are safe.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
attn_status attn_bwd_noalloc(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                             const float* LSE, void* dQ, void* dK, void* dV,
                             int B, int H, int S, int D, float scale, int causal,
                             const attn_opts* opts, void* stream);

/*
 * Split-KV forward pass: the same O and LSE as attn_fwd, computed by splitting
 * the keys into chunks that run as separate workgroups and merging the
 * per-chunk results by their log-sum-exp,
 *     LSE = ln sum_c exp(LSE_c),   O = sum_c exp(LSE_c - LSE) O_c,
 * which is exact for softmax over disjoint key sets.  It gives a long key
 * sequence with few query rows (decoding, chunked prefill) enough
 * workgroups to fill the GPU.  The pages motivate the LSE output by long
 * sequences (page "FlashAttention-4: Algorithm and Kernel Pipelining
 * Co-Design for Asymmetric Hardware Scaling", abstract; page
 * "FlashAttention-3 и FlashAttention-4", section "Режим 2-CTA MMA"); the
 * split itself is not on the pages.
 *   in : Q bf16 [B,H,Sq,D]; K, V bf16 [B,H,Sk,D]
 *   out: O bf16 [B,H,Sq,D]; LSE fp32 [B,H,Sq]
 *   Sq and Sk may differ.  causal != 0 reads the queries as the last Sq of
 *   the Sk positions: key j is hidden from query i when j > i + Sk - Sq
 *   (requires Sk >= Sq, else ATTN_ERR_SHAPE; Sq == Sk is attn_fwd's mask).
 *   num_splits: number of key chunks, >= 1, clamped to the number of key
 *   tiles; 0 chooses one that gives about two workgroups per compute unit.
 *   Sq == 1 (decoding) runs a dedicated kernel: fp32 dot products, no
 *   matrix tiles, native exp2 whatever opts->exp_mode says.
 *   workspace: caller-owned device memory of at least
 *   attn_fwd_splitkv_workspace_bytes(...) bytes (same arguments), 256-byte
 *   aligned, holding the per-chunk fp32 outputs and LSEs; contents on entry
 *   do not matter.  Two calls in flight at once must not share it.
 *   Errors: as attn_fwd, plus ATTN_ERR_VALUE for num_splits < 0 and
 *   ATTN_ERR_WORKSPACE for a missing, small or misaligned workspace.
 */
size_t attn_fwd_splitkv_workspace_bytes(int B, int H, int Sq, int Sk, int D, int causal, int num_splits);
attn_status attn_fwd_splitkv(const void* Q, const void* K, const void* V, void* O, float* LSE,
                             void* workspace, size_t workspace_bytes,
                             int B, int H, int Sq, int Sk, int D, float scale, int causal,
                             int num_splits, const attn_opts* opts, void* stream);

/* Human-readable text of a status code (static storage). */
const char* attn_strerror(attn_status s);

/*
 * FP8 forward pass with incoherent processing (D = 128 only).  Page
 * "FlashAttention-3 и FlashAttention-4", section "Поддержка FP8 с контролем
 * ошибок": before the rounding to FP8, Q and K pass a cheap transform that
 * spreads outlier values over the coordinates, which lowers the FP8 error.
 * The transform here is x -> (x * signs) H / sqrt(128), H the 128 x 128
 * Sylvester-Hadamard matrix (orthogonal, so Q K^T is unchanged).  The
 * format is OCP FP8 E4M3 (largest value 448, round to nearest even); the
 * scales are per Q row, per (batch, head) for K and per V column, none of
 * them tied to a tile of the kernel.
 *
 * Two calls: attn_fp8_quantize fills a caller-owned buffer with the
 * quantized operands, attn_fwd_fp8 computes O and LSE from it.  A buffer
 * can serve several attn_fwd_fp8 calls (e.g. both causal settings).
 *
 * Buffer: attn_fp8_buffer_bytes(B, H, S, D) bytes, 256-byte aligned, holding
 * seven regions at the byte offsets attn_fp8_buffer_offsets writes (each
 * rounded up to 256 bytes); Sp = S rounded up to 128, rows past S are zero:
 *   [0] q8  uint8 [B*H, Sp, 128]  E4M3 codes of the transformed Q
 *   [1] k8  uint8 [B*H, Sp, 128]  E4M3 codes of the transformed K
 *   [2] v8t uint8 [B*H, 128, Sp]  E4M3 codes of V, transposed; inside each
 *           group of 64 keys, key 32 kb + 8 r + 4 h + e (kb, h in {0,1};
 *           r, e in 0..3) is stored at position 32 h + 16 kb + 4 r + e
 *   [3] qs  fp32 [B*H, Sp]        one scale per Q row
 *   [4] ks  fp32 [B*H]            one scale per (batch, head) for K
 *   [5] vs  fp32 [B*H, 128]       one scale per V column
 *   [6] scratch (V's column maxima, K's head maxima)
 * A value x is represented as scale * e4m3(code); each scale is the
 * group's max |x| / 448 (1 for an all-zero group), and each code is the
 * float64 quotient x * 448 / max|x| rounded to nearest E4M3 (ties to even).
 */
size_t attn_fp8_buffer_bytes(int B, int H, int S, int D);
attn_status attn_fp8_buffer_offsets(int B, int H, int S, int D, size_t offsets[7]);

/*
 *   in : Q, K, V bf16 [B,H,S,D] (D = 128); signs: device fp32 [128] of +1 / -1
 *        (the random signs of the transform), or NULL for no transform
 *        (plain FP8 quantization of Q and K)
 *   out: buf as above (its previous contents do not matter)
 *   Errors: ATTN_ERR_NULL, ATTN_ERR_SHAPE, ATTN_ERR_UNSUPPORTED (D != 128),
 *   ATTN_ERR_ALIGN (inputs not 16-byte aligned), ATTN_ERR_WORKSPACE (buf
 *   missing, small or not 256-byte aligned), ATTN_ERR_HIP.
 */
attn_status attn_fp8_quantize(const void* Q, const void* K, const void* V, const float* signs, void* buf,
                              size_t buf_bytes, int B, int H, int S, int D, void* stream);

/*
 * Forward pass from a quantized buffer: the online softmax of attn_fwd with
 * S = scale * Q8 K8^T and O += P8 V8, P rounded to E4M3 per key tile of 64
 * (relative to the running row max), the row sum taken over the unrounded P;
 * O = acc / l (bf16), LSE = m + ln l (fp32, natural log).
 *   in : buf from attn_fp8_quantize with the same B, H, S, D
 *   out: O bf16 [B,H,S,D]; LSE fp32 [B,H,S]
 *   opts: rescale_tau as in attn_fwd, but at most 8 is applied (P is rounded
 *   to E4M3, whose largest value is 448, and unnormalised probabilities stay
 *   below 2^tau); exp_mode and bwd_mode are ignored.
 *   Errors: as attn_fp8_quantize, plus ATTN_ERR_VALUE for a non-finite scale.
 */
attn_status attn_fwd_fp8(const void* buf, size_t buf_bytes, void* O, float* LSE, int B, int H, int S, int D,
                         float scale, int causal, const attn_opts* opts, void* stream);

/*
 * Diagnostic: the FP8 forward's score product on given E4M3 codes.  For
 * each of nblk blocks, C = A B with A 32 x 128 codes (row-major), B 128 x 32
 * codes passed transposed as Bt (32 x 128, row-major) and C 32 x 32 fp32
 * (row-major), computed by the same two chained v_mfma_f32_32x32x64_f8f6f4
 * and operand layout as one 32 x 32 block of S = Q K^T at D = 128.  A, Bt, C
 * are device pointers of nblk * 4096, nblk * 4096 bytes and nblk * 1024
 * floats, 16-byte aligned; nblk = 0 launches nothing.  Codes 0x7F and 0xFF
 * (NaN) give NaN.  Errors: ATTN_ERR_NULL, ATTN_ERR_SHAPE (nblk < 0),
 * ATTN_ERR_ALIGN, ATTN_ERR_HIP.
 */
attn_status attn_fp8_dot_eval(const void* A, const void* Bt, float* C, long nblk, void* stream);

/*
 * Diagnostic: evaluate the kernels' exp2 on n fp32 values, y[i] = 2^x[i],
 * with the same device code the forward kernel uses for mode (an
 * attn_exp_mode).  x and y are device pointers of n floats (n >= 0; n = 0
 * launches nothing).  Arguments below the clamp point (-127) return the
 * value at the clamp point in ATTN_EXP_POLY mode.
 */
attn_status attn_exp2_eval(const float* x, float* y, long n, int mode, void* stream);

/*
 * Diagnostic: select a kernel variant kept for measurement, for subsequent
 * calls in this process.  kernel: "fwd" (D = 128 forward: 0 default, 1 the
 * eight-wavefront tile at every length, 2 the four-wavefront tile at every
 * length), "bwd_dq" (D = 128 dQ of the split backward: 0 default, 1 four
 * wavefronts per workgroup, 2 eight, at every length), "bwd_dkdv" (D = 64
 * and 256 dK / dV of the split backward: 0 default, the pipelined tile;
 * 1 the one-pass tile); variant -1 returns to the choice of the
 * environment variables ATTN97_FWD_VARIANT / ATTN97_DQ_VARIANT /
 * ATTN97_DKDV_VARIANT (default 0).  Every variant computes the same result.
 * The choice is process-global state shared by every thread and stream of
 * the process; it is not synchronised, so set it only while no other thread
 * calls the library.
 * Errors: ATTN_ERR_NULL, ATTN_ERR_UNSUPPORTED (unknown kernel name),
 * ATTN_ERR_VALUE (variant out of range).
 */
attn_status attn_set_variant(const char* kernel, int variant);

/*
 * Timing of the library's own kernels, for measurement tools.  While enabled,
 * every kernel launch is bracketed by two hipEvents recorded on the launch
 * stream.  attn_prof_collect synchronises on those events and returns, for
 * the kernel named `kernel` ("fwd", "bwd_pre", "bwd_main", "bwd_dq", "bwd_dkdv",
 * "dq_convert", "fwd_splitkv", "splitkv_merge", "fp8_quantize" (all three
 * kernels of attn_fp8_quantize), "fwd_fp8"), the number of launches and the
 * summed milliseconds since the last reset.  Events are created on first use
 * and kept; at most 65536 launches are recorded between resets (later ones
 * are not timed).  The enable flag and the event pool are process-global
 * state, not synchronised: meant for a single-threaded benchmark driver, and
 * while timing is enabled the library is not safe to call from several
 * threads.  With timing disabled (the default) the library keeps no state.
 */
attn_status attn_prof_enable(int on);
attn_status attn_prof_reset(void);
attn_status attn_prof_collect(const char* kernel, int* count, double* total_ms);

/* Library version string. */
const char* attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN97_H */

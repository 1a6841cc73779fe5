/*
 * puro_fp8.h -- C ABI of the blockwise-scaled FP8 linear-layer library (MI355X / gfx950).
 *
 * The method: the main linear layers of a Transformer run their matmuls in FP8 with
 * fine-grained block scaling after DeepSeek-V3, while numerically sensitive work and
 * master weights / optimizer state stay in BF16 / FP32 (ModelScope write-up
 * "清华开源 Puro-2B：4400 美元训练，15 项任务平均指标超 Qwen2-1.5B！", section
 * 精度: FP8 分块量化与净效率收益).  Activations are grouped by 128 and weights use
 * 128x128 blocks (agihunt digest "清华用消费级 5090 花 6890 美元从零训 2B，15 项均分超过
 * Qwen2", section 方法 / Method, FP8 bullet); each block carries its own scale so that
 * one outlier does not inflate a scale shared by the whole tensor (same digest,
 * section 术语 / glossary, "blockwise FP8").
 *
 * Numerics fixed by this library where the pages are silent:
 *   - FP8 format: OCP E4M3 (bias 7, largest finite 448, NaN = S.1111.111, no inf).
 *   - Per tile: amax = max|x| (exact, from the bf16 input); amax_eff = max(amax, 2^-96);
 *     scale s = fl32(amax_eff / 448) (stored); r = fl32(448 / amax_eff);
 *     code = E4M3(fl32(x * r)) with round-to-nearest-even, saturating at 448, sign kept.
 *     Both divisions are correctly rounded fp32 divisions.
 *   - GEMM: for every 128-deep contraction slice kb, the FP8 products are accumulated in
 *     fp32 (matrix cores) and then added, multiplied by sA(i,kb) * sB(j,kb), into a
 *     separate fp32 accumulator; the result is written as bf16 (round to nearest even)
 *     or fp32.  Exact result: C[i,j] = sum_k dec(A[i,k]) sA(i,k/128) dec(B[j,k]) sB(j,k/128).
 *   - Non-finite input is outside the bit-exact contract: a NaN in a tile makes its scale
 *     and codes NaN; an infinity gives that tile's scale +inf.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers (HIP device memory); the caller owns every
 *     buffer; the library allocates nothing and keeps no per-call state.
 *   - Matrices are row-major; a leading dimension ("ld") is the distance, in ELEMENTS of
 *     that buffer's type, between consecutive rows; ld >= row width.
 *   - Pointers must be 16-byte aligned and ld * element_size must be a multiple of 16.
 *   - Work is enqueued asynchronously on the caller's stream `st` (NULL = the null stream);
 *     nothing synchronizes.  Device faults surface at the caller's next synchronization.
 *   - Every argument check runs on the host before any HIP call; a failed check returns a
 *     negative status and launches nothing.  A dimension of 0 is a no-op returning
 *     PURO_OK.  After a launch, a HIP launch error is reported as PURO_ERR_HIP.
 *   - Thread-safe: concurrent calls on different streams are independent.
 */
#ifndef PURO_FP8_H
#define PURO_FP8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;

enum {
  PURO_OK = 0,
  PURO_ERR_NULLPTR = -1,     /* a required pointer is NULL, or exactly one of an optional pair */
  PURO_ERR_SHAPE = -2,       /* a dimension is negative or not a multiple of 128 where required */
  PURO_ERR_ALIGN = -3,       /* a pointer is not 16-byte aligned */
  PURO_ERR_LD = -4,          /* ld < width, or ld * element size not a multiple of 16 bytes */
  PURO_ERR_MODE = -5,        /* unknown GEMM mode */
  PURO_ERR_DTYPE = -6,       /* unknown output dtype */
  PURO_ERR_WORKSPACE = -7,   /* workspace smaller than puro_fp8_gemm_workspace_size() */
  PURO_ERR_HIP = -8,         /* the HIP runtime reported an error at launch */
  PURO_ERR_UNSUPPORTED = -9  /* valid request this library does not implement (e.g. a size limit) */
};

enum { PURO_GEMM_FWD = 0, PURO_GEMM_DGRAD = 1, PURO_GEMM_WGRAD = 2 };
enum { PURO_OUT_BF16 = 0, PURO_OUT_FP32 = 1 };

/*
 * 1x128 activation quantizer (forward X, dgrad dY).  Groups of 128 consecutive features
 * of one row share a scale (agihunt digest, section 方法, FP8 bullet: activations grouped
 * by 128; the group runs along the GEMM's contraction axis).
 *   x   : bf16 [M, K], row stride ldx (elements); K % 128 == 0; M >= 0 arbitrary.
 *   q   : uint8 E4M3 codes [M, K], row stride ldq (bytes).
 *   s   : fp32 scales, contraction-block-major [K/128][M] (contiguous, stride M): s[kb*M + m]
 *         is the scale of row m, columns 128kb .. 128kb+127.
 */
int puro_fp8_quant_act_1x128(const void* x, int64_t M, int64_t K, int64_t ldx,
                             uint8_t* q, int64_t ldq, float* s, hipStream_t st);

/*
 * 128x1 activation / gradient quantizer for the wgrad operands, written transposed.
 * Groups of 128 consecutive tokens of one column share a scale (the wgrad contraction
 * runs over tokens; same passages as above).
 *   x   : bf16 [T, C], row stride ldx (elements); T % 128 == 0; C % 8 == 0.
 *   qT  : uint8 codes [C, T] (token-contiguous), row stride ldqT (bytes).
 *   sT  : fp32 scales [T/128][C] (contiguous, stride C): sT[tb*C + c] is the scale of
 *         column c, tokens 128tb .. 128tb+127.
 */
int puro_fp8_quant_act_128x1(const void* x, int64_t T, int64_t C, int64_t ldx,
                             uint8_t* qT, int64_t ldqT, float* sT, hipStream_t st);

/*
 * Dual quantizer: one read of x yields exactly what puro_fp8_quant_act_1x128(x) and
 * puro_fp8_quant_act_128x1(x) write (same bytes, same scales).  In training, X and dY each
 * feed one GEMM with 1x128 groups (FWD / DGRAD) and one with 128x1 groups (WGRAD), so both
 * quantizations of the same tensor are needed (same passages as above).
 *   x   : bf16 [T, C], row stride ldx (elements); T % 128 == 0; C % 128 == 0.
 *   q   : uint8 codes [T, C], row stride ldq (bytes); s: fp32 [C/128][T] (1x128 layout).
 *   qT  : uint8 codes [C, T], row stride ldqT (bytes); sT: fp32 [T/128][C] (128x1 layout).
 * All four outputs are required.
 */
int puro_fp8_quant_act_dual(const void* x, int64_t T, int64_t C, int64_t ldx,
                            uint8_t* q, int64_t ldq, float* s,
                            uint8_t* qT, int64_t ldqT, float* sT, hipStream_t st);

/*
 * 128x128 weight-block quantizer (agihunt digest, section 方法, FP8 bullet: weights in
 * 128x128 blocks), with an optional transposed copy for dgrad.
 *   w   : bf16 [N, K], row stride ldw (elements); N % 128 == 0, K % 128 == 0.
 *   q   : uint8 codes [N, K], row stride ldq (bytes).
 *   s   : fp32 scales [N/128][K/128] row-major.
 *   qT  : optional uint8 codes [K, N], row stride ldqT: qT[k][n] == q[n][k].
 *   sT  : optional fp32 scales [K/128][N/128]: sT[kb][nb] == s[nb][kb].
 *   qT and sT are both NULL or both non-NULL (else PURO_ERR_NULLPTR).
 */
int puro_fp8_quant_w_128x128(const void* w, int64_t N, int64_t K, int64_t ldw,
                             uint8_t* q, int64_t ldq, float* s,
                             uint8_t* qT, int64_t ldqT, float* sT, hipStream_t st);

/*
 * One weight of puro_fp8_quant_w_128x128_batch: the arguments of puro_fp8_quant_w_128x128, with
 * the same meaning, layouts and rules.
 */
typedef struct puro_fp8_wq_job {
  const void* w;
  int64_t N, K, ldw;
  uint8_t* q;
  int64_t ldq;
  float* s;
  uint8_t* qT;   /* optional, with sT */
  int64_t ldqT;
  float* sT;
} puro_fp8_wq_job;

/*
 * Several 128x128 weight quantizations in one launch.  Every job writes exactly the bytes that
 * puro_fp8_quant_w_128x128 with its arguments writes.  The weights of a layer do not depend on
 * the activations, and the pages train with BF16/FP32 master weights (agihunt digest, section
 * 方法, FP8 bullet), so all of a layer's weights are quantized anew after each optimizer step:
 * one launch then replaces one small launch per weight.
 *   jobs   : host array of n_jobs descriptors (read before the call returns; not kept).
 *   n_jobs : 0 .. 16 (else PURO_ERR_UNSUPPORTED); 0 does nothing.
 * Every job is checked as puro_fp8_quant_w_128x128 checks its arguments before anything is
 * launched; the first failing job's error is returned and nothing runs.  Jobs must not write
 * overlapping outputs.
 */
int puro_fp8_quant_w_128x128_batch(const puro_fp8_wq_job* jobs, int n_jobs, hipStream_t st);

/*
 * Blockwise-scaled FP8 GEMM  C[M,N] = sum_kb sA(i,kb) sB(j,kb) sum_{k in kb} dec(A[i,k]) dec(B[j,k]).
 * ModelScope write-up, section 精度 (FP8 matmuls of the main linear layers, DeepSeek-V3
 * block scaling); per-slice fp32 promotion into a separate fp32 accumulator.
 *   mode: PURO_GEMM_FWD   Y  = X  W^T : A = Xq   [T, Din],  B = Wq  [Dout, Din]
 *         PURO_GEMM_DGRAD dX = dY W   : A = dYq  [T, Dout], B = WqT [Din, Dout]
 *         PURO_GEMM_WGRAD dW = dY^T X : A = dYqT [Dout, T], B = XqT [Din, T]
 *   A   : uint8 codes [M, K], row stride lda (bytes); sA: fp32 [K/128][M].
 *   B   : uint8 codes [N, K], row stride ldb (bytes);
 *         sB: FWD/DGRAD fp32 [N/128][K/128] (128x128 blocks); WGRAD fp32 [K/128][N].
 *   C   : [M, N] bf16 (out_dtype PURO_OUT_BF16) or fp32 (PURO_OUT_FP32), row stride ldc
 *         (elements).  M, N, K must be multiples of 128 (else PURO_ERR_SHAPE).
 *         lda and ldb must not exceed 2^29 bytes (else PURO_ERR_UNSUPPORTED).
 *   workspace / workspace_bytes: scratch the caller provides; must be at least
 *         puro_fp8_gemm_workspace_size(mode, M, N, K) bytes (may be NULL when that is 0).
 *         That size covers every launch the call makes (a call may run its leading rows
 *         unsplit and the rest with a contraction split); it is checked in full before the
 *         first launch, so a too-small workspace fails with nothing written.
 *   The summation order inside the GEMM is not part of the contract.
 */
int puro_fp8_gemm(int mode, int64_t M, int64_t N, int64_t K,
                  const uint8_t* A, int64_t lda, const float* sA,
                  const uint8_t* B, int64_t ldb, const float* sB,
                  void* C, int64_t ldc, int out_dtype,
                  void* workspace, size_t workspace_bytes, hipStream_t st);

/*
 * Accumulating variant, fp32 output only: C[i,j] = fl32(C[i,j] + P[i,j]), where P is exactly the
 * fp32 result puro_fp8_gemm writes for the same arguments (one fp32 addition per element).
 * For accumulating the fp32 weight gradient over micro-batches: the pages keep master weights
 * and optimizer state in BF16/FP32 (agihunt digest, section 方法, FP8 bullet) and train with a
 * global batch of 1536 sequences of 4096 tokens (same section, training layout), far more
 * tokens than one WGRAD call takes.  Arguments, layouts and errors as puro_fp8_gemm, with
 * out_dtype fixed to PURO_OUT_FP32; C is read and written.  K == 0 leaves C unchanged.
 */
int puro_fp8_gemm_accumulate(int mode, int64_t M, int64_t N, int64_t K,
                             const uint8_t* A, int64_t lda, const float* sA,
                             const uint8_t* B, int64_t ldb, const float* sB,
                             float* C, int64_t ldc,
                             void* workspace, size_t workspace_bytes, hipStream_t st);

/*
 * GEMM with the 1x128 quantization of its output fused into the epilogue: C (bf16, as
 * puro_fp8_gemm with PURO_OUT_BF16 writes it) and, from those bf16 values, exactly what
 * puro_fp8_quant_act_1x128(C) would write: codes q [M, N] (row stride ldq bytes) and scales
 * s [N/128][M].  For an output that feeds the next FP8 linear layer as its activation (groups
 * of 128 along that layer's contraction axis, agihunt digest, section 方法, FP8 bullet), this
 * saves re-reading C.  Arguments, layouts and errors as puro_fp8_gemm; q and s are required.
 */
int puro_fp8_gemm_quant(int mode, int64_t M, int64_t N, int64_t K,
                        const uint8_t* A, int64_t lda, const float* sA,
                        const uint8_t* B, int64_t ldb, const float* sB,
                        void* C, int64_t ldc, uint8_t* q, int64_t ldq, float* s,
                        void* workspace, size_t workspace_bytes, hipStream_t st);

/*
 * Allocation-free puro_fp8_gemm, for callers that cannot allocate device memory or pass a
 * workspace (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, layouts, result and errors as puro_fp8_gemm, except the
 * workspace: the contraction split's fp32 partial sums go to a device buffer of
 * PURO_FP8_SCRATCH_BYTES that the library owns, one per device, held from the library's
 * first use on that device until the process ends.  A problem with
 * puro_fp8_gemm_workspace_size(mode, M, N, K) > PURO_FP8_SCRATCH_BYTES is refused with
 * PURO_ERR_WORKSPACE before anything is launched.  The call itself allocates nothing.
 * Every call on one device shares that buffer: calls that may overlap on the same device
 * (different streams without ordering between them) race and must be serialized by the
 * caller.  The buffer needs no initialization; each call writes every partial it reads.
 */
#define PURO_FP8_SCRATCH_BYTES (64u * 1024u * 1024u)
int puro_fp8_gemm_noalloc(int mode, int64_t M, int64_t N, int64_t K,
                          const uint8_t* A, int64_t lda, const float* sA,
                          const uint8_t* B, int64_t ldb, const float* sB,
                          void* C, int64_t ldc, int out_dtype, hipStream_t st);

/* Bytes of workspace puro_fp8_gemm, puro_fp8_gemm_accumulate and puro_fp8_gemm_quant need (0 = none):
 * the largest fp32 partial-sum buffer of any launch the call makes. */
size_t puro_fp8_gemm_workspace_size(int mode, int64_t M, int64_t N, int64_t K);

/*
 * MXFP8 variant.  On Blackwell the pages' linear layers run MXFP8 instead of the 1x128 /
 * 128x128 scheme (agihunt digest, section 方法, FP8 bullet); the pages give no detail, so the
 * format is the OCP Microscaling (MX) one with E4M3 elements:
 *   - blocks of 32 consecutive elements along the consuming GEMM's contraction axis;
 *   - one E8M0 scale byte per block, X = 2^(code - 127) (code 255 = NaN), chosen as
 *     2^(floor(log2 amax) - 8) (8 = exponent of E4M3's largest normal, 448 = 1.75 * 2^8),
 *     clamped to [2^-127, 2^127]; an all-zero block gets code 0;
 *   - elements E4M3_rne_sat(x / X) (x / X is exact; values in [448, 512) X saturate).
 *   - a block holding a NaN or an infinity gets code 255 and NaN element codes
 *     (outside the bit-exact contract, as for the blockwise quantizers).
 * Scale layout, for an operand [R, K] whose blocks run along K: bytes [K/128][R][4]; byte
 * (kb, r, j) scales row r, elements 128 kb + 32 j .. 128 kb + 32 j + 31.
 */

/*
 * MX dual quantizer: one read of x bf16 [T, C] yields
 *   q  : codes [T, C] (row stride ldq), blocks along C; xs : scales [C/128][T][4];
 *   qT : codes [C, T] (row stride ldqT), blocks along T; xsT: scales [T/128][C][4].
 * Activations and gradients use both (FWD / DGRAD and WGRAD); for a weight W [Dout, Din],
 * q serves FWD and qT (blocks along Dout) serves DGRAD.  T % 128 == 0, C % 128 == 0.
 */
int puro_fp8_mx_quant_dual(const void* x, int64_t T, int64_t C, int64_t ldx,
                           uint8_t* q, int64_t ldq, uint8_t* xs,
                           uint8_t* qT, int64_t ldqT, uint8_t* xsT, hipStream_t st);

/*
 * MX GEMM  C[M,N] = sum_k dec(A[i,k]) X_A(i, k/32) dec(B[j,k]) X_B(j, k/32), accumulated in fp32
 * by the matrix cores, which apply the block scales themselves (no separate promotion).
 *   A : codes [M, K] (row stride lda), xa: scales [K/128][M][4];
 *   B : codes [N, K] (row stride ldb), xb: scales [K/128][N][4];
 *   C, out_dtype, workspace: as puro_fp8_gemm (workspace from puro_fp8_mx_gemm_workspace_size).
 * FWD / DGRAD / WGRAD differ only in which quantized tensors are passed.
 */
int puro_fp8_mx_gemm(int64_t M, int64_t N, int64_t K,
                     const uint8_t* A, int64_t lda, const uint8_t* xa,
                     const uint8_t* B, int64_t ldb, const uint8_t* xb,
                     void* C, int64_t ldc, int out_dtype,
                     void* workspace, size_t workspace_bytes, hipStream_t st);

/* Bytes of workspace puro_fp8_mx_gemm needs for this problem (0 = none). */
size_t puro_fp8_mx_gemm_workspace_size(int64_t M, int64_t N, int64_t K);

/*
 * Verification helper: the device fp32 -> E4M3 cast every quantizer uses
 * (round-to-nearest-even, saturating at 448, sign kept, NaN -> NaN code), applied
 * elementwise: q[i] = E4M3(v[i]) for 0 <= i < n.  v and q must be 16-byte aligned.
 */
int puro_fp8_cast_e4m3(const float* v, int64_t n, uint8_t* q, hipStream_t st);

/* Human-readable text of a status code (static storage). */
const char* puro_fp8_strerror(int status);

/* Library version: major * 10000 + minor * 100 + patch. */
int puro_fp8_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PURO_FP8_H */

// C-ABI layer: argument validation on the host, then one asynchronous launch on the
// caller's stream.  Every check runs before any HIP call; a failed check launches nothing.
#include "../../include/puro_fp8.h"

#include <hip/hip_runtime_api.h>

#include "internal.hpp"

namespace {

constexpr int64_t kGroup = 128;
constexpr int64_t kIntMax = 0x7FFFFFFF;
constexpr int kModeMx = 3;   // the MXFP8 GEMM's internal mode (not a public PURO_GEMM_* value)
// Largest operand row stride (bytes) of the GEMM: the kernels form each lane's copy offset inside
// an 8-row group, 7 * ld + 127, in 32 bits.
constexpr int64_t kMaxGemmLd = int64_t(1) << 29;

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// a * b > INT32_MAX for non-negative a, b (without overflowing): one workgroup per tile must fit a
// one-dimensional grid
inline bool too_many_blocks(int64_t a, int64_t b) { return a > 0 && b > kIntMax / a; }

inline int from_hip(hipError_t e) {
  if (e == hipErrorInvalidConfiguration) return PURO_ERR_UNSUPPORTED;
  return e == hipSuccess ? PURO_OK : PURO_ERR_HIP;
}

}  // namespace

extern "C" {

int puro_fp8_quant_act_1x128(const void* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q, int64_t ldq,
                             float* s, hipStream_t st) {
  if (M < 0 || K < 0) return PURO_ERR_SHAPE;
  if (K % kGroup) return PURO_ERR_SHAPE;
  if (M == 0 || K == 0) return PURO_OK;
  if (!x || !q || !s) return PURO_ERR_NULLPTR;
  if (!aligned16(x) || !aligned16(q) || !aligned16(s)) return PURO_ERR_ALIGN;
  if (ldx < K || ldq < K || (ldx * 2) % 16 || ldq % 16) return PURO_ERR_LD;
  if (K / kGroup > kIntMax) return PURO_ERR_UNSUPPORTED;
  return from_hip(puro::launch_quant_1x128(x, M, K, ldx, q, ldq, s, st));
}

int puro_fp8_quant_act_128x1(const void* x, int64_t T, int64_t C, int64_t ldx, uint8_t* qT, int64_t ldqT,
                             float* sT, hipStream_t st) {
  if (T < 0 || C < 0) return PURO_ERR_SHAPE;
  if (T % kGroup || C % 8) return PURO_ERR_SHAPE;
  if (T == 0 || C == 0) return PURO_OK;
  if (!x || !qT || !sT) return PURO_ERR_NULLPTR;
  if (!aligned16(x) || !aligned16(qT) || !aligned16(sT)) return PURO_ERR_ALIGN;
  if (ldx < C || ldqT < T || (ldx * 2) % 16 || ldqT % 16) return PURO_ERR_LD;
  if (too_many_blocks(T / kGroup, (C + 63) / 64)) return PURO_ERR_UNSUPPORTED;
  return from_hip(puro::launch_quant_128x1(x, T, C, ldx, qT, ldqT, sT, st));
}

int puro_fp8_quant_act_dual(const void* x, int64_t T, int64_t C, int64_t ldx, uint8_t* q, int64_t ldq,
                            float* s, uint8_t* qT, int64_t ldqT, float* sT, hipStream_t st) {
  if (T < 0 || C < 0) return PURO_ERR_SHAPE;
  if (T % kGroup || C % kGroup) return PURO_ERR_SHAPE;
  if (T == 0 || C == 0) return PURO_OK;
  if (!x || !q || !s || !qT || !sT) return PURO_ERR_NULLPTR;
  if (!aligned16(x) || !aligned16(q) || !aligned16(s) || !aligned16(qT) || !aligned16(sT)) return PURO_ERR_ALIGN;
  if (ldx < C || ldq < C || ldqT < T || (ldx * 2) % 16 || ldq % 16 || ldqT % 16) return PURO_ERR_LD;
  if (too_many_blocks(T / kGroup, C / kGroup)) return PURO_ERR_UNSUPPORTED;
  return from_hip(puro::launch_quant_dual(x, T, C, ldx, q, ldq, s, qT, ldqT, sT, st));
}

// Argument checks of one 128x128 weight quantization (PURO_OK also for an empty weight).
static int check_quant_w(const void* w, int64_t N, int64_t K, int64_t ldw, const uint8_t* q, int64_t ldq,
                         const float* s, const uint8_t* qT, int64_t ldqT, const float* sT) {
  if (N < 0 || K < 0) return PURO_ERR_SHAPE;
  if (N % kGroup || K % kGroup) return PURO_ERR_SHAPE;
  if ((qT == nullptr) != (sT == nullptr)) return PURO_ERR_NULLPTR;
  if (N == 0 || K == 0) return PURO_OK;
  if (!w || !q || !s) return PURO_ERR_NULLPTR;
  if (!aligned16(w) || !aligned16(q) || !aligned16(s)) return PURO_ERR_ALIGN;
  if (qT && (!aligned16(qT) || !aligned16(sT))) return PURO_ERR_ALIGN;
  if (ldw < K || ldq < K || (ldw * 2) % 16 || ldq % 16) return PURO_ERR_LD;
  if (qT && (ldqT < N || ldqT % 16)) return PURO_ERR_LD;
  if (too_many_blocks(N / kGroup, K / kGroup)) return PURO_ERR_UNSUPPORTED;
  return PURO_OK;
}

int puro_fp8_quant_w_128x128(const void* w, int64_t N, int64_t K, int64_t ldw, uint8_t* q, int64_t ldq,
                             float* s, uint8_t* qT, int64_t ldqT, float* sT, hipStream_t st) {
  const int rc = check_quant_w(w, N, K, ldw, q, ldq, s, qT, ldqT, sT);
  if (rc != PURO_OK || N == 0 || K == 0) return rc;
  return from_hip(puro::launch_quant_128x128(w, N, K, ldw, q, ldq, s, qT, ldqT, sT, st));
}

int puro_fp8_quant_w_128x128_batch(const puro_fp8_wq_job* jobs, int n_jobs, hipStream_t st) {
  if (n_jobs < 0 || n_jobs > puro::kMaxWeightJobs) return PURO_ERR_UNSUPPORTED;
  if (n_jobs == 0) return PURO_OK;
  if (!jobs) return PURO_ERR_NULLPTR;
  puro::WeightJob b[puro::kMaxWeightJobs];
  int64_t blocks = 0;
  for (int i = 0; i < n_jobs; ++i) {
    const puro_fp8_wq_job& j = jobs[i];
    const int rc = check_quant_w(j.w, j.N, j.K, j.ldw, j.q, j.ldq, j.s, j.qT, j.ldqT, j.sT);
    if (rc != PURO_OK) return rc;
    b[i] = puro::WeightJob{static_cast<const uint16_t*>(j.w), j.N, j.K, j.ldw, j.q, j.ldq, j.s, j.qT, j.ldqT, j.sT,
                           0, 0};
    blocks += (j.N / kGroup) * (j.K / kGroup);
  }
  if (blocks > 0x7FFFFFFF) return PURO_ERR_UNSUPPORTED;
  return from_hip(puro::launch_quant_128x128_batch(b, n_jobs, st));
}

static_assert(PURO_FP8_SCRATCH_BYTES == puro::kScratchBytes, "the header's scratch size is the library's");

// use_scratch: the library's own device buffer replaces the caller's workspace (allocation-free
// entry point); a problem whose partials exceed it is refused before any HIP call.
static int gemm_common(int mode, int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda, const float* sA,
                       const uint8_t* B, int64_t ldb, const float* sB, void* C, int64_t ldc, int out_dtype,
                       bool accumulate, void* workspace, size_t workspace_bytes, hipStream_t st,
                       bool quant = false, uint8_t* q = nullptr, int64_t ldq = 0, float* qs = nullptr,
                       bool use_scratch = false) {
  if (mode != PURO_GEMM_FWD && mode != PURO_GEMM_DGRAD && mode != PURO_GEMM_WGRAD && mode != kModeMx)
    return PURO_ERR_MODE;
  if (out_dtype != PURO_OUT_BF16 && out_dtype != PURO_OUT_FP32) return PURO_ERR_DTYPE;
  if (M < 0 || N < 0 || K < 0) return PURO_ERR_SHAPE;
  if (M % kGroup || N % kGroup || K % kGroup) return PURO_ERR_SHAPE;
  if (M == 0 || N == 0) return PURO_OK;
  const int64_t es = out_dtype == PURO_OUT_BF16 ? 2 : 4;
  if (!C) return PURO_ERR_NULLPTR;
  if (!aligned16(C)) return PURO_ERR_ALIGN;
  if (ldc < N || (ldc * es) % 16) return PURO_ERR_LD;
  if (quant) {
    if (!q || !qs) return PURO_ERR_NULLPTR;
    if (!aligned16(q) || !aligned16(qs)) return PURO_ERR_ALIGN;
    if (ldq < N || ldq % 16) return PURO_ERR_LD;
  }
  if (K > 0) {
    if (!A || !B || !sA || !sB) return PURO_ERR_NULLPTR;
    if (!aligned16(A) || !aligned16(B) || !aligned16(sA) || !aligned16(sB)) return PURO_ERR_ALIGN;
    if (lda < K || ldb < K || lda % 16 || ldb % 16) return PURO_ERR_LD;
  }
  if (M > kIntMax || N > kIntMax || K > kIntMax) return PURO_ERR_UNSUPPORTED;
  if (K > 0 && (lda > kMaxGemmLd || ldb > kMaxGemmLd)) return PURO_ERR_UNSUPPORTED;
  const size_t need = puro::gemm_workspace_bytes(mode, M, N, K);
  if (use_scratch) {
    if (need > puro::kScratchBytes) return PURO_ERR_WORKSPACE;
    workspace = nullptr;
    workspace_bytes = 0;
    if (need > 0) {
      if (puro::scratch_buffer(&workspace) != hipSuccess) return PURO_ERR_HIP;
      workspace_bytes = puro::kScratchBytes;
    }
  }
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return PURO_ERR_WORKSPACE;
  return from_hip(puro::launch_gemm(mode, M, N, K, A, lda, sA, B, ldb, sB, C, ldc, out_dtype == PURO_OUT_BF16,
                                    accumulate, quant ? q : nullptr, ldq, qs, workspace, workspace_bytes, st));
}

int puro_fp8_gemm(int mode, int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda, const float* sA,
                  const uint8_t* B, int64_t ldb, const float* sB, void* C, int64_t ldc, int out_dtype,
                  void* workspace, size_t workspace_bytes, hipStream_t st) {
  if (mode == kModeMx) return PURO_ERR_MODE;   // internal mode: puro_fp8_mx_gemm
  return gemm_common(mode, M, N, K, A, lda, sA, B, ldb, sB, C, ldc, out_dtype, false, workspace, workspace_bytes,
                     st);
}

int puro_fp8_gemm_noalloc(int mode, int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                          const float* sA, const uint8_t* B, int64_t ldb, const float* sB, void* C, int64_t ldc,
                          int out_dtype, hipStream_t st) {
  if (mode == kModeMx) return PURO_ERR_MODE;
  return gemm_common(mode, M, N, K, A, lda, sA, B, ldb, sB, C, ldc, out_dtype, false, nullptr, 0, st, false,
                     nullptr, 0, nullptr, true);
}

int puro_fp8_gemm_quant(int mode, int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda, const float* sA,
                        const uint8_t* B, int64_t ldb, const float* sB, void* C, int64_t ldc, uint8_t* q, int64_t ldq,
                        float* s, void* workspace, size_t workspace_bytes, hipStream_t st) {
  if (mode == kModeMx) return PURO_ERR_MODE;
  return gemm_common(mode, M, N, K, A, lda, sA, B, ldb, sB, C, ldc, PURO_OUT_BF16, false, workspace, workspace_bytes,
                     st, true, q, ldq, s);
}

int puro_fp8_mx_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda, const uint8_t* xa,
                     const uint8_t* B, int64_t ldb, const uint8_t* xb, void* C, int64_t ldc, int out_dtype,
                     void* workspace, size_t workspace_bytes, hipStream_t st) {
  return gemm_common(kModeMx, M, N, K, A, lda, reinterpret_cast<const float*>(xa), B, ldb,
                     reinterpret_cast<const float*>(xb), C, ldc, out_dtype, false, workspace, workspace_bytes, st);
}

size_t puro_fp8_mx_gemm_workspace_size(int64_t M, int64_t N, int64_t K) {
  return puro::gemm_workspace_bytes(kModeMx, M, N, K);
}

int puro_fp8_mx_quant_dual(const void* x, int64_t T, int64_t C, int64_t ldx, uint8_t* q, int64_t ldq, uint8_t* xs,
                           uint8_t* qT, int64_t ldqT, uint8_t* xsT, hipStream_t st) {
  if (T < 0 || C < 0) return PURO_ERR_SHAPE;
  if (T % kGroup || C % kGroup) return PURO_ERR_SHAPE;
  if (T == 0 || C == 0) return PURO_OK;
  if (!x || !q || !xs || !qT || !xsT) return PURO_ERR_NULLPTR;
  if (!aligned16(x) || !aligned16(q) || !aligned16(xs) || !aligned16(qT) || !aligned16(xsT)) return PURO_ERR_ALIGN;
  if (ldx < C || ldq < C || ldqT < T || (ldx * 2) % 16 || ldq % 16 || ldqT % 16) return PURO_ERR_LD;
  if (too_many_blocks(T / kGroup, C / kGroup)) return PURO_ERR_UNSUPPORTED;
  return from_hip(puro::launch_mx_quant_dual(x, T, C, ldx, q, ldq, xs, qT, ldqT, xsT, st));
}

int puro_fp8_gemm_accumulate(int mode, int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                             const float* sA, const uint8_t* B, int64_t ldb, const float* sB, float* C, int64_t ldc,
                             void* workspace, size_t workspace_bytes, hipStream_t st) {
  if (mode == kModeMx) return PURO_ERR_MODE;   // internal mode: no accumulating MX entry point
  return gemm_common(mode, M, N, K, A, lda, sA, B, ldb, sB, C, ldc, PURO_OUT_FP32, true, workspace,
                     workspace_bytes, st);
}

size_t puro_fp8_gemm_workspace_size(int mode, int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  return puro::gemm_workspace_bytes(mode, M, N, K);
}

int puro_fp8_cast_e4m3(const float* v, int64_t n, uint8_t* q, hipStream_t st) {
  if (n < 0) return PURO_ERR_SHAPE;
  if (n == 0) return PURO_OK;
  if (!v || !q) return PURO_ERR_NULLPTR;
  if (!aligned16(v) || !aligned16(q)) return PURO_ERR_ALIGN;
  return from_hip(puro::launch_cast_e4m3(v, n, q, st));
}

const char* puro_fp8_strerror(int status) {
  switch (status) {
    case PURO_OK: return "ok";
    case PURO_ERR_NULLPTR: return "null pointer (or only one of an optional pointer pair)";
    case PURO_ERR_SHAPE: return "bad shape (negative, or not a multiple of 128 where required)";
    case PURO_ERR_ALIGN: return "pointer not 16-byte aligned";
    case PURO_ERR_LD: return "bad leading dimension (smaller than the row, or not a multiple of 16 bytes)";
    case PURO_ERR_MODE: return "unknown GEMM mode";
    case PURO_ERR_DTYPE: return "unknown output dtype";
    case PURO_ERR_WORKSPACE: return "workspace too small";
    case PURO_ERR_HIP: return "HIP runtime error at launch";
    case PURO_ERR_UNSUPPORTED: return "request outside what this library implements";
    default: return "unknown status";
  }
}

int puro_fp8_version(void) { return 100; }

}  // extern "C"

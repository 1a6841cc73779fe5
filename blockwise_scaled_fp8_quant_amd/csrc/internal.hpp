// Internal launcher declarations between the C-ABI layer (abi.cpp) and the kernels.
// Shapes and pointers are validated by the caller before any of these runs.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace puro {

// s[kb * lds + m] is the scale of row m, group kb; lds = 0 means M (the public layout).
hipError_t launch_quant_1x128(const void* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q,
                              int64_t ldq, float* s, hipStream_t st, int64_t lds = 0);
hipError_t launch_quant_128x1(const void* x, int64_t T, int64_t C, int64_t ldx, uint8_t* qT,
                              int64_t ldqT, float* sT, hipStream_t st);
hipError_t launch_quant_dual(const void* x, int64_t T, int64_t C, int64_t ldx, uint8_t* q, int64_t ldq,
                             float* s, uint8_t* qT, int64_t ldqT, float* sT, hipStream_t st);
hipError_t launch_mx_quant_dual(const void* x, int64_t T, int64_t C, int64_t ldx, uint8_t* q, int64_t ldq,
                                uint8_t* xs, uint8_t* qT, int64_t ldqT, uint8_t* xsT, hipStream_t st);
hipError_t launch_quant_128x128(const void* w, int64_t N, int64_t K, int64_t ldw, uint8_t* q,
                                int64_t ldq, float* s, uint8_t* qT, int64_t ldqT, float* sT,
                                hipStream_t st);
hipError_t launch_cast_e4m3(const float* v, int64_t n, uint8_t* q, hipStream_t st);

// Several 128x128 weight quantizations in one launch (each exactly as launch_quant_128x128).
// bt and first are filled in by the launcher.
struct WeightJob {
  const uint16_t* w;
  int64_t N, K, ldw;
  uint8_t* q;
  int64_t ldq;
  float* s;
  uint8_t* qT;     // optional (with sT)
  int64_t ldqT;
  float* sT;
  int bt;          // token-run length of the job's tile order
  int64_t first;   // the job's first block in the launch
};
constexpr int kMaxWeightJobs = 16;
struct WeightJobs {
  WeightJob job[kMaxWeightJobs];
  int n;
};
hipError_t launch_quant_128x128_batch(const WeightJob* jobs, int n, hipStream_t st);

// GEMM: mode 0 FWD, 1 DGRAD, 2 WGRAD, 3 MXFP8 (E8M0 block scales, bytes [K/128][rows][4]);
// out_bf16 selects bf16 (else fp32) output; accumulate (fp32 output only) adds the result to
// C; q / ldq / qs (bf16 output only, optional) also write the 1x128 quantization of the bf16
// C along N (codes [M, N], scales [N/128][M]).
size_t gemm_workspace_bytes(int mode, int64_t M, int64_t N, int64_t K);

// The library's own split-K buffer for callers that cannot allocate: a file-scope device array of
// kScratchBytes per device (the same figure as PURO_FP8_SCRATCH_BYTES).  scratch_buffer returns the
// current device's copy (its address is looked up once per device).  Every call on a device shares
// it, so calls that overlap on one device race.
constexpr size_t kScratchBytes = size_t(64) << 20;
hipError_t scratch_buffer(void** ptr);

// The launches of one GEMM call, in order: part p covers rows row0 .. row0 + rows - 1 of A and C
// with the contraction split into `splits` ranges (1 = unsplit).  Returns the number of parts
// (1 or 2); gemm_workspace_bytes is the largest part_workspace of the plan.
struct GemmPart {
  int64_t row0, rows;
  int splits;
};
int gemm_parts(int64_t M, int64_t N, int64_t K, GemmPart parts[2]);
size_t part_workspace(const GemmPart& p, int64_t N);
hipError_t launch_gemm(int mode, int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                       const float* sA, const uint8_t* B, int64_t ldb, const float* sB, void* C,
                       int64_t ldc, bool out_bf16, bool accumulate, uint8_t* q, int64_t ldq, float* qs,
                       void* workspace, size_t workspace_bytes, hipStream_t st);

}  // namespace puro

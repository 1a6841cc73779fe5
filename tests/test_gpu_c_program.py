"""The C ABI driven from a plain C program on the GPU, without PyTorch: buffers from hipMalloc,
a stream from hipStreamCreate (default priority), results copied back with hipMemcpy.

Checked inside the program (it exits non-zero on the first mismatch):
  * the dual quantizer writes exactly the bytes of the 1x128 and 128x1 quantizers;
  * a FWD GEMM on codes of small integers with power-of-two scales equals, bit for bit, the
    exact result the program sums in double (every partial sum is an integer multiple of a
    power of two far inside fp32's range);
  * a call with an invalid leading dimension returns PURO_ERR_LD and leaves its output alone.
The E4M3 codes used are the OCP format's encodings of 0, +-1, +-2, +-3, +-4 (0x00, 0x38/0xB8,
0x40/0xC0, 0x44/0xC4, 0x48/0xC8).
"""
import os
import shutil
import subprocess

import pytest

from gpu_util import say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "blockwise_scaled_fp8_quant_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

PROGRAM = r"""
#define __HIP_PLATFORM_AMD__
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include "puro_fp8.h"

#define CHECK(x) do { if ((x) != hipSuccess) { printf("HIP error at line %d\n", __LINE__); return 90; } } while (0)

static unsigned seed = 12345u;
static unsigned next(void) { seed = seed * 1664525u + 1013904223u; return seed >> 8; }

int main(void) {
  enum { M = 256, K = 512, N = 384 };
  static const unsigned char codes[9] = {0x00, 0x38, 0xB8, 0x40, 0xC0, 0x44, 0xC4, 0x48, 0xC8};
  static const double values[9] = {0, 1, -1, 2, -2, 3, -3, 4, -4};
  hipStream_t st;
  unsigned short* hx = malloc(sizeof(unsigned short) * M * K);
  unsigned char *ha = malloc(M * K), *hb = malloc(N * K), *h1 = malloc(M * K), *h2 = malloc(M * K);
  float *hsa = malloc(sizeof(float) * (K / 128) * M), *hsb = malloc(sizeof(float) * (N / 128) * (K / 128));
  float *hc = malloc(sizeof(float) * M * N), *f1 = malloc(sizeof(float) * M * K), *f2 = malloc(sizeof(float) * M * K);
  void *x, *q, *s, *qT, *sT, *q1, *s1, *qT1, *sT1, *A, *B, *sA, *sB, *C;
  int i, j, k, kb, bad = 0;
  CHECK(hipStreamCreate(&st));

  /* bf16 input: random signs and magnitudes over a few binades (the bits are built directly) */
  for (i = 0; i < M * K; ++i)
    hx[i] = (unsigned short)(((next() & 1u) << 15) | ((112u + next() % 32u) << 7) | (next() & 0x7Fu));
  CHECK(hipMalloc(&x, sizeof(unsigned short) * M * K));
  CHECK(hipMalloc(&q, M * K)); CHECK(hipMalloc(&qT, M * K)); CHECK(hipMalloc(&q1, M * K)); CHECK(hipMalloc(&qT1, M * K));
  CHECK(hipMalloc(&s, sizeof(float) * M * K / 128)); CHECK(hipMalloc(&sT, sizeof(float) * M * K / 128));
  CHECK(hipMalloc(&s1, sizeof(float) * M * K / 128)); CHECK(hipMalloc(&sT1, sizeof(float) * M * K / 128));
  CHECK(hipMemcpy(x, hx, sizeof(unsigned short) * M * K, hipMemcpyHostToDevice));
  if (puro_fp8_quant_act_dual(x, M, K, K, q, K, s, qT, M, sT, st) != PURO_OK) return 1;
  if (puro_fp8_quant_act_1x128(x, M, K, K, q1, K, s1, st) != PURO_OK) return 2;
  if (puro_fp8_quant_act_128x1(x, M, K, K, qT1, M, sT1, st) != PURO_OK) return 3;
  CHECK(hipStreamSynchronize(st));
  CHECK(hipMemcpy(h1, q, M * K, hipMemcpyDeviceToHost)); CHECK(hipMemcpy(h2, q1, M * K, hipMemcpyDeviceToHost));
  if (memcmp(h1, h2, M * K)) return 4;
  CHECK(hipMemcpy(h1, qT, M * K, hipMemcpyDeviceToHost)); CHECK(hipMemcpy(h2, qT1, M * K, hipMemcpyDeviceToHost));
  if (memcmp(h1, h2, M * K)) return 5;
  CHECK(hipMemcpy(f1, s, sizeof(float) * M * K / 128, hipMemcpyDeviceToHost));
  CHECK(hipMemcpy(f2, s1, sizeof(float) * M * K / 128, hipMemcpyDeviceToHost));
  if (memcmp(f1, f2, sizeof(float) * M * K / 128)) return 6;
  CHECK(hipMemcpy(f1, sT, sizeof(float) * M * K / 128, hipMemcpyDeviceToHost));
  CHECK(hipMemcpy(f2, sT1, sizeof(float) * M * K / 128, hipMemcpyDeviceToHost));
  if (memcmp(f1, f2, sizeof(float) * M * K / 128)) return 7;

  /* FWD GEMM on small-integer codes with power-of-two scales: exact */
  int* ia = malloc(sizeof(int) * M * K);
  int* ib = malloc(sizeof(int) * N * K);
  for (i = 0; i < M * K; ++i) { ia[i] = (int)(next() % 9u); ha[i] = codes[ia[i]]; }
  for (i = 0; i < N * K; ++i) { ib[i] = (int)(next() % 9u); hb[i] = codes[ib[i]]; }
  for (i = 0; i < (K / 128) * M; ++i) hsa[i] = (float)(1 << (next() % 4u)) / 4.0f;       /* 1/4 .. 2 */
  for (i = 0; i < (N / 128) * (K / 128); ++i) hsb[i] = (float)(1 << (next() % 3u)) / 2.0f; /* 1/2 .. 2 */
  CHECK(hipMalloc(&A, M * K)); CHECK(hipMalloc(&B, N * K));
  CHECK(hipMalloc(&sA, sizeof(float) * (K / 128) * M)); CHECK(hipMalloc(&sB, sizeof(float) * (N / 128) * (K / 128)));
  CHECK(hipMalloc(&C, sizeof(float) * M * N));
  CHECK(hipMemcpy(A, ha, M * K, hipMemcpyHostToDevice)); CHECK(hipMemcpy(B, hb, N * K, hipMemcpyHostToDevice));
  CHECK(hipMemcpy(sA, hsa, sizeof(float) * (K / 128) * M, hipMemcpyHostToDevice));
  CHECK(hipMemcpy(sB, hsb, sizeof(float) * (N / 128) * (K / 128), hipMemcpyHostToDevice));
  if (puro_fp8_gemm_workspace_size(PURO_GEMM_FWD, M, N, K) != 0) return 8;
  if (puro_fp8_gemm(PURO_GEMM_FWD, M, N, K, A, K, sA, B, K, sB, C, N, PURO_OUT_FP32, NULL, 0, st) != PURO_OK) return 9;
  CHECK(hipStreamSynchronize(st));
  CHECK(hipMemcpy(hc, C, sizeof(float) * M * N, hipMemcpyDeviceToHost));
  for (i = 0; i < M; ++i)
    for (j = 0; j < N; ++j) {
      double acc = 0.0;
      for (kb = 0; kb < K / 128; ++kb) {
        double part = 0.0;
        for (k = kb * 128; k < kb * 128 + 128; ++k) part += values[ia[i * K + k]] * values[ib[j * K + k]];
        acc += part * hsa[kb * M + i] * hsb[(j / 128) * (K / 128) + kb];
      }
      if ((double)hc[i * N + j] != acc) ++bad;
    }
  if (bad) { printf("%d GEMM outputs differ from the exact sum\n", bad); return 10; }

  /* an invalid leading dimension is rejected before anything runs */
  for (i = 0; i < M * N; ++i) hc[i] = 7.0f;
  CHECK(hipMemcpy(C, hc, sizeof(float) * M * N, hipMemcpyHostToDevice));
  if (puro_fp8_gemm(PURO_GEMM_FWD, M, N, K, A, K - 16, sA, B, K, sB, C, N, PURO_OUT_FP32, NULL, 0, st) != PURO_ERR_LD)
    return 11;
  CHECK(hipStreamSynchronize(st));
  CHECK(hipMemcpy(hc, C, sizeof(float) * M * N, hipMemcpyDeviceToHost));
  for (i = 0; i < M * N; ++i) if (hc[i] != 7.0f) return 12;

  CHECK(hipStreamDestroy(st));
  hipFree(x); hipFree(q); hipFree(s); hipFree(qT); hipFree(sT); hipFree(q1); hipFree(s1); hipFree(qT1); hipFree(sT1);
  hipFree(A); hipFree(B); hipFree(sA); hipFree(sB); hipFree(C);
  printf("ok\n");
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_c_program_on_the_gpu(tmp_path):
    src = tmp_path / "gpu_prog.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "gpu_prog"
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROCM, "include"), str(src), "-o", str(exe),
           "-L", PKG, "-lpuro_fp8", f"-Wl,-rpath,{PKG}", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    say("[c program] running the C-ABI program on the GPU")
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, f"exit {run.returncode}: {run.stdout} {run.stderr}"
    assert run.stdout.strip().endswith("ok"), run.stdout

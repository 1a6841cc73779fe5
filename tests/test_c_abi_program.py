"""The C ABI from C itself (no GPU needed): include/puro_fp8.h compiles as strict C11 with
every warning an error, a C program links against libpuro_fp8.so, and the host-side checks
answer as the header documents (they run before any HIP call, so nothing is launched)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "blockwise_scaled_fp8_quant_amd")
LIB = os.path.join(PKG, "libpuro_fp8.so")

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "puro_fp8.h"

int main(void) {
  puro_fp8_wq_job job;
  size_t ws;
  memset(&job, 0, sizeof job);
  if (puro_fp8_version() < 100) return 1;
  /* argument checks: the documented status, and no HIP call before it */
  if (puro_fp8_quant_act_1x128(NULL, 128, 128, 128, NULL, 128, NULL, NULL) != PURO_ERR_NULLPTR) return 2;
  if (puro_fp8_quant_act_1x128(NULL, 128, 100, 128, NULL, 128, NULL, NULL) != PURO_ERR_SHAPE) return 3;
  if (puro_fp8_quant_act_dual(NULL, -128, 128, 128, NULL, 128, NULL, NULL, 128, NULL, NULL) != PURO_ERR_SHAPE) return 4;
  if (puro_fp8_gemm(7, 128, 128, 128, NULL, 128, NULL, NULL, 128, NULL, NULL, 128, PURO_OUT_BF16, NULL, 0, NULL)
      != PURO_ERR_MODE) return 5;
  if (puro_fp8_gemm(PURO_GEMM_FWD, 128, 128, 128, NULL, 128, NULL, NULL, 128, NULL, NULL, 128, 5, NULL, 0, NULL)
      != PURO_ERR_DTYPE) return 6;
  /* an empty problem is a no-op */
  if (puro_fp8_gemm(PURO_GEMM_FWD, 0, 128, 128, NULL, 128, NULL, NULL, 128, NULL, NULL, 128, PURO_OUT_BF16, NULL, 0,
                    NULL) != PURO_OK) return 7;
  if (puro_fp8_quant_w_128x128_batch(&job, 17, NULL) != PURO_ERR_UNSUPPORTED) return 8;
  if (puro_fp8_quant_w_128x128_batch(NULL, 0, NULL) != PURO_OK) return 9;
  ws = puro_fp8_gemm_workspace_size(PURO_GEMM_WGRAD, 2048, 2048, 16384);
  if (ws == 0 || ws % (2048u * 2048u * 4u) != 0) return 10;
  if (puro_fp8_mx_gemm_workspace_size(0, 128, 128) != 0) return 11;
  printf("ok %d [%s] %zu\n", puro_fp8_version(), puro_fp8_strerror(PURO_ERR_SHAPE), ws);
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_header_compiles_as_c_and_a_c_program_links_and_runs(tmp_path):
    assert os.path.exists(LIB), "build the library first (python blockwise_scaled_fp8_quant_amd/build.py)"
    src = tmp_path / "prog.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "prog"
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
           str(src), "-o", str(exe), "-L", PKG, "-lpuro_fp8", f"-Wl,-rpath,{PKG}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, f"exit {run.returncode}: {run.stdout} {run.stderr}"
    assert run.stdout.startswith("ok "), run.stdout

"""The GEMM's launch plan against its workspace query (CPU only; nothing is launched).

A call runs as one or two launches ("parts": an unsplit leading block of whole tile rows, then the
remaining rows with a contraction split of their own).  The workspace the caller is told to
provide (puro_fp8_gemm_workspace_size) must cover every part, for every entry point that follows
the plan, so that the library can check it in full before the first launch.

A C++ program links libpuro_fp8.so, walks a grid of shapes (every M that is a multiple of 128 up
to 32768 against a set of N and K, plus named shapes where a remainder needs a larger split than
the whole problem would), and checks for each: the parts tile the rows exactly, in order; every
part's partial-sum bytes fit in the queried workspace; the query equals the largest part (no
over-asking); and the public query returns the internal figure.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "blockwise_scaled_fp8_quant_amd")
LIB = os.path.join(PKG, "libpuro_fp8.so")

PROGRAM = r"""
#include <cstdio>
#include <cstdint>
#include "internal.hpp"
#include "puro_fp8.h"

static int check(int64_t M, int64_t N, int64_t K, long* n_split_parts) {
  puro::GemmPart parts[2];
  const int n = puro::gemm_parts(M, N, K, parts);
  if (n < 1 || n > 2) return 1;
  const size_t ws = puro::gemm_workspace_bytes(2, M, N, K);
  for (int mode = 0; mode < 3; ++mode)
    if (puro_fp8_gemm_workspace_size(mode, M, N, K) != ws) return 2;
  int64_t next = 0;
  size_t largest = 0;
  for (int i = 0; i < n; ++i) {
    if (parts[i].row0 != next || parts[i].rows <= 0 || parts[i].rows % 128) return 3;
    if (parts[i].splits < 1 || parts[i].splits > 8) return 4;
    next += parts[i].rows;
    const size_t need = puro::part_workspace(parts[i], N);
    if (need > ws) {
      std::printf("part %d of %lld x %lld x %lld needs %zu > %zu\n", i, (long long)M, (long long)N,
                  (long long)K, need, ws);
      return 5;
    }
    if (need != (parts[i].splits > 1 ? (size_t)parts[i].splits * parts[i].rows * N * 4 : 0)) return 6;
    if (need > largest) largest = need;
    if (parts[i].splits > 1) ++*n_split_parts;
  }
  if (next != M) return 7;
  if (largest != ws) return 8;
  return 0;
}

int main() {
  const int64_t Ns[] = {128, 256, 384, 1024, 2048, 4096, 6144, 8192, 12288, 16384};
  const int64_t Ks[] = {128, 1024, 2048, 4096, 8192, 16384, 32768, 65536};
  long cases = 0, split_parts = 0;
  for (int64_t M = 128; M <= 32768; M += 128)
    for (int64_t N : Ns)
      for (int64_t K : Ks) {
        const int rc = check(M, N, K, &split_parts);
        if (rc) { std::printf("FAIL %d at %lld %lld %lld\n", rc, (long long)M, (long long)N, (long long)K); return rc; }
        ++cases;
      }
  // shapes whose remainder rows need a larger split than the whole problem
  const int64_t named[][3] = {{11008, 2048, 32768}, {2816, 8192, 32768}, {11264, 2048, 32768},
                              {12288, 2048, 16384}, {8448, 2048, 16384}};
  for (auto& s : named) {
    const int rc = check(s[0], s[1], s[2], &split_parts);
    if (rc) { std::printf("FAIL %d at named %lld %lld %lld\n", rc, (long long)s[0], (long long)s[1], (long long)s[2]); return rc; }
    puro::GemmPart parts[2];
    std::printf("named %lld x %lld x %lld: %d part(s)", (long long)s[0], (long long)s[1], (long long)s[2],
                puro::gemm_parts(s[0], s[1], s[2], parts));
    for (int i = 0; i < puro::gemm_parts(s[0], s[1], s[2], parts); ++i)
      std::printf(" [rows %lld, splits %d]", (long long)parts[i].rows, parts[i].splits);
    std::printf(", workspace %zu\n", puro::gemm_workspace_bytes(2, s[0], s[1], s[2]));
  }
  std::printf("ok %ld shapes, %ld split parts\n", cases, split_parts);
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("g++") is None, reason="no C++ compiler")
def test_workspace_query_covers_every_launch_of_the_plan(tmp_path):
    assert os.path.exists(LIB), "build the library first (python blockwise_scaled_fp8_quant_amd/build.py)"
    src = tmp_path / "plan.cpp"
    src.write_text(PROGRAM)
    exe = tmp_path / "plan"
    cmd = ["g++", "-std=c++17", "-O1", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"), str(src), "-o", str(exe),
           "-L", PKG, "-lpuro_fp8", f"-Wl,-rpath,{PKG}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    print(run.stdout)
    assert run.returncode == 0, f"exit {run.returncode}: {run.stdout} {run.stderr}"
    assert "ok " in run.stdout
    # the named shapes all take the two-part plan
    assert run.stdout.count("2 part(s)") >= 3, run.stdout

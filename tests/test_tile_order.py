"""The GEMM kernels' workgroup-to-tile order (block_of in gemm_args.hpp), checked on the host.

A program compiled host-only from the kernels' own header walks a grid of tile counts, contraction
splits and group sizes and checks that the order is a bijection of the launch grid onto
(split, tile row, tile column) -- every output tile of every split is computed exactly once -- and
that it keeps the locality it is for: the workgroups the dispatcher places on one XCD (workgroup b
on XCD b % 8) share one split wherever the grid allows it, and on the layer sweep's WGRAD launches
the 32 workgroups an XCD runs at once touch at most 12 operand panels (tile rows plus tile columns).
It also checks the four-wave kernels' L2 prefetch row selection (pf_row): each lane's row stays in
its own run of lanes, and over the tiles that share a panel every row is fetched exactly once.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "blockwise_scaled_fp8_quant_amd", "csrc")
HIPCC = shutil.which("hipcc") or ("/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else None)

PROGRAM = r"""
#include <cstdio>
#include <set>
#include <vector>
#include "gemm_args.hpp"

static int check(int tiles_m, int tiles_n, int splits, int group) {
  const int nt = tiles_m * tiles_n, total = nt * splits;
  std::vector<int> seen((size_t)total, 0);
  std::vector<std::set<int>> xcd_splits(8);
  for (int b = 0; b < total; ++b) {
    int s, tm, tn;
    puro::block_of(b, tiles_m, tiles_n, splits, group, s, tm, tn);
    if (s < 0 || s >= splits || tm < 0 || tm >= tiles_m || tn < 0 || tn >= tiles_n) return 1;
    if (seen[(size_t)s * nt + (size_t)tm * tiles_n + tn]++) return 2;
    xcd_splits[b % 8].insert(s);
  }
  // a run of total / 8 workgroups per XCD covers run / nt splits, or lies inside one
  if (total % 8 == 0) {
    const int run = total / 8;
    const size_t most = run >= nt ? (size_t)(run / nt) + (run % nt ? 1 : 0) : (nt % run == 0 ? 1 : 2);
    for (auto& xs : xcd_splits)
      if (xs.size() > most) return 3;
  }
  return 0;
}

// operand panels (distinct tile rows + tile columns) of the first `resident` workgroups per XCD
static int panels(int tiles_m, int tiles_n, int splits, int group, int resident) {
  int worst = 0;
  for (int x = 0; x < 8; ++x) {
    std::set<long> rows, cols;
    int n = 0;
    for (int b = x; b < tiles_m * tiles_n * splits && n < resident; b += 8, ++n) {
      int s, tm, tn;
      puro::block_of(b, tiles_m, tiles_n, splits, group, s, tm, tn);
      rows.insert((long)s * 100000 + tm);
      cols.insert((long)s * 100000 + tn);
    }
    const int p = (int)(rows.size() + cols.size());
    if (p > worst) worst = p;
  }
  return worst;
}

int main() {
  long cases = 0;
  for (int tm = 1; tm <= 40; ++tm)
    for (int tn = 1; tn <= 40; ++tn)
      for (int sp : {1, 2, 4, 8})
        for (int g : {1, 4, 8}) {
          const int rc = check(tm, tn, sp, g);
          if (rc) { std::printf("FAIL %d at tiles %d x %d, splits %d, group %d\n", rc, tm, tn, sp, g); return rc; }
          ++cases;
        }
  // the layer sweep's WGRAD launches at 16384 tokens (256 x 256 tiles, with the group the library
  // picks): qkv 4096 x 2048 in 2 splits, o 2048 x 2048 in 4, gate_up 12288 x 2048 as 8192 rows
  // unsplit plus 4096 rows in 2 (group 8), down 2048 x 6144 unsplit (group 4)
  const int sweep[][5] = {{16, 8, 2, 8, 12}, {8, 8, 4, 8, 12}, {32, 8, 1, 8, 12}, {16, 8, 2, 8, 12}, {8, 24, 1, 4, 10}};
  for (auto& s : sweep) {
    const int p = panels(s[0], s[1], s[2], s[3], 32);
    std::printf("tiles %d x %d splits %d group %d: %d panels per XCD\n", s[0], s[1], s[2], s[3], p);
    if (p > s[4]) return 10;
  }
  // the L2 prefetch's row selection: a lane's row stays in its own run of n lanes (so inside the
  // wave's 64 rows), and over the n tiles that share a panel (tile classes 0 .. n - 1) every row
  // of the wave is fetched exactly once
  for (int n : {1, 2, 4, 8}) {
    if (puro::pf_share(n) != n) return 20;
    for (int base = 0; base < 64; base += n) {
      int hits[64] = {0};
      for (int tile = base; tile < base + n; ++tile) {
        std::set<int> rows;
        for (int lane = 0; lane < 64; ++lane) {
          const int r = puro::pf_row(lane, tile, n);
          if (r < (lane & ~(n - 1)) || r >= (lane & ~(n - 1)) + n) return 21;
          rows.insert(r);
        }
        if ((int)rows.size() != 64 / n) return 22;
        for (int r : rows) ++hits[r];
      }
      for (int r = 0; r < 64; ++r)
        if (hits[r] != 1) return 23;
    }
  }
  for (int v : {3, 5, 6, 7, 9, 16, 32}) {
    const int s = puro::pf_share(v);
    if (s > v || (s & (s - 1)) || s > 8) return 24;
  }
  // shares of the sweep's FWD (group 4: 8 tiles share an A panel, 4 a B panel) and WGRAD launches
  puro::GemmArgs g{};
  g.group = 4; g.tiles_m = 64; g.tiles_n = 16;
  if (puro::pf_share_a(g) != 8 || puro::pf_share_b(g) != 4) return 25;
  g.group = 8; g.tiles_m = 16; g.tiles_n = 8;
  if (puro::pf_share_a(g) != 4 || puro::pf_share_b(g) != 8) return 26;
  g.group = 4; g.tiles_m = 1; g.tiles_n = 2;
  if (puro::pf_share_a(g) != 2 || puro::pf_share_b(g) != 1) return 27;
  std::printf("ok %ld cases\n", cases);
  return 0;
}
"""


@pytest.mark.skipif(HIPCC is None, reason="no hipcc")
def test_block_order_is_a_bijection_with_xcd_locality(tmp_path):
    src = tmp_path / "order.cpp"
    src.write_text(PROGRAM)
    exe = tmp_path / "order"
    cmd = [HIPCC, "-x", "hip", "--cuda-host-only", "-std=c++17", "-O1", "-I", CSRC, str(src), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    print(run.stdout)
    assert run.returncode == 0, f"exit {run.returncode}: {run.stdout} {run.stderr}"
    assert "ok " in run.stdout

// Arguments and helpers shared by the two blockwise GEMM kernels (gemm.hip: eight waves, 64x128 wave
// tiles, every mode; gemm_w4.hip: four waves, 128x128 wave tiles, FWD and DGRAD).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace puro {

typedef uint32_t g_u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t g_u32x2 __attribute__((ext_vector_type(2)));
typedef float g_f32x4 __attribute__((ext_vector_type(4)));

// Two fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32), packed low | high << 16.
typedef __bf16 g_bf16x2 __attribute__((ext_vector_type(2)));
typedef float g_f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
  const g_f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, g_bf16x2));
}

struct GemmArgs {
  int M, N, K;
  int tiles_m, tiles_n;
  int group;             // tile rows walked together (see block_of)
  int splits;            // contraction split: block b works on split b / (tiles_m * tiles_n)
  int kb_per_split;      // 128-deep slices per split
  int64_t split_stride;  // elements between the fp32 partial outputs of consecutive splits
  const uint8_t* A;
  int64_t lda;
  const float* sA;
  int64_t ldsa;          // elements (MX: 4-byte rows) between consecutive slices of sA: M, or the
                         // full problem's M when this launch covers a range of its rows
  const uint8_t* B;
  int64_t ldb;
  const float* sB;
  void* C;
  int64_t ldc;
  int accumulate;        // fp32 output only: C = C + result (one fp32 add per element)
  uint8_t* q;            // bf16 output only, optional: 1x128 quantization of C along N
  int64_t ldq;
  float* qs;             // its scales: qs[nb * ldqs + i] for row i, column block nb
  int64_t ldqs;
};

// Map the linear workgroup id to (split, tile_m, tile_n).  The dispatcher places workgroup b on XCD
// b % 8; each XCD gets a contiguous run of the split-major tile sequence, so with a contraction
// split the workgroups of one XCD share their split's slice range rather than each running a
// piece of every split.  Within a split the sequence walks `group` tile rows at a time across all
// tile columns: an XCD's run is then a compact block of tiles whose A rows and B columns its
// workgroups read from the XCD's L2 (B is also shared between XCDs through the memory-side cache).
__host__ __device__ inline void block_of(int b, int tiles_m, int tiles_n, int splits, int group, int& split,
                                         int& tm, int& tn) {
  const int nt = tiles_m * tiles_n;
  const int total = nt * splits;
  const int full = (total >> 3) << 3;
  int logical = b;
  if (b < full) logical = (b & 7) * (total >> 3) + (b >> 3);
  split = logical / nt;
  const int t = logical - split * nt;
  const int per_group = group * tiles_n;
  const int g = t / per_group;
  const int first_m = g * group;
  const int gsize = tiles_m - first_m < group ? tiles_m - first_m : group;
  const int r = t - g * per_group;
  tm = first_m + r % gsize;
  tn = r / gsize;
}

// Which rows a wave's L2 prefetch of a later slice touches (four-wave kernels).  The workgroups an
// XCD runs at once form a block of `group` tile rows by 32 / group tile columns (block_of), and each line only has to reach that
// XCD's L2 once: an A row panel is shared by the block's tiles of one tile row (n_a of them, told
// apart by tile column mod n_a), a B panel by its tiles of one tile column (n_b, by tile row mod
// n_b).  So of each run of n lanes (n = n_a or n_b) only one row is fetched, the one whose class
// is the tile's: the lanes of the run all point at it and their requests merge into one line.
__host__ __device__ inline int pf_share(int n) { return n >= 8 ? 8 : n >= 4 ? 4 : n >= 2 ? 2 : 1; }
__host__ __device__ inline int pf_share_a(const GemmArgs& p) {
  return pf_share(32 / p.group < p.tiles_n ? 32 / p.group : p.tiles_n);
}
__host__ __device__ inline int pf_share_b(const GemmArgs& p) { return pf_share(p.group < p.tiles_m ? p.group : p.tiles_m); }
__host__ __device__ inline int pf_row(int lane, int tile, int n) { return (lane & ~(n - 1)) + (tile & (n - 1)); }

hipError_t launch_w4(const GemmArgs& a, bool out_bf16, hipStream_t st);
// Whether launch_w4 can take these arguments: its operand offsets are 32-bit buffer offsets.
bool w4_supported(const GemmArgs& a);
// The MXFP8 GEMM in the four-wave form (E8M0 block scales in sA / sB), and its offset check.
hipError_t launch_w4mx(const GemmArgs& a, bool out_bf16, hipStream_t st);
bool w4mx_supported(const GemmArgs& a);

}  // namespace puro

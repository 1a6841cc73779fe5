// gfx950 blockwise-scaled FP8 GEMM with per-128-slice fp32 promotion.
//
//   C[i,j] = sum_kb  sA(i,kb) * sB(j,kb) * P_kb[i,j],   P_kb[i,j] = sum_{k in slice kb} A[i,k] B[j,k]
//
// P_kb is produced by the FP8 matrix cores (v_mfma_f32_32x32x64_f8f6f4, E4M3 x E4M3 ->
// fp32; two instructions cover one 128-deep slice of a 32x32 output tile), and the
// promotion C_acc += P_kb * (sA * sB) runs on the vector ALUs into a separate fp32
// accumulator, following the DeepSeek-V3-style fine-grained scheme the pages adopt
// (ModelScope write-up on Puro-2B, section 精度).
//
// Kernel shape (one workgroup = 512 threads = 8 waves, one 256x256 output tile):
//  * K loop over 128-deep slices, double-buffered in LDS (2 x 66 KB): the next slice's
//    A and B tiles (256 x 128 bytes each) and its scales are copied HBM/L2 -> LDS with
//    global_load_lds_dwordx4 (no VGPR round trip) while the current slice is multiplied.
//  * LDS rows are 128 bytes = 8 chunks of 16 bytes; chunk c of row r is stored at
//    position c ^ ((r >> 1) & 7) so that the fragment reads of 16 consecutive rows spread
//    over all 64 LDS banks.  The swizzle is applied on the global side: the lane that
//    lands at position p fetches logical chunk p ^ ((r >> 1) & 7).
//  * Waves form a 4 (M) x 2 (N) grid of 64 x 128 wave tiles: 2 x 4 MFMA tiles of 32x32,
//    128 fp32 accumulator registers per lane.
//  * Operand roles inside the MFMA are swapped (the B fragment is the instruction's A
//    operand) so that every lane owns ONE output row and 16 output columns: the row
//    scale sA(i,kb) is one register per lane and slice; with 128x128 weight blocks
//    (FWD/DGRAD) the whole scale product is one multiply per lane and slice, and the
//    promotion is one FMA per accumulator element per slice.
//  * Tiles are visited in an XCD-aware order: the dispatcher places workgroup b on XCD
//    b % 8, so each XCD is given a contiguous run of tiles, walked in groups of 4 or 8 tile
//    rows (choose_group), so that the tiles resident in one XCD's L2 share A rows and B
//    columns.
//  * The epilogue stages each wave's output tile in LDS and writes whole row segments
//    with 16-byte stores (a lane's own fragment holds one row of a 32x32 tile, as 4 runs
//    of 4 adjacent columns).
//  * M or N that are multiples of 128 but not of 256 leave half-empty edge tiles: their
//    loads are clamped to valid rows and their stores are masked.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>

#include "codec.hpp"
#include "gemm_args.hpp"
#include "internal.hpp"
#include "gemm_slice_asm.inc"

namespace puro {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

constexpr int kBM = 256, kBN = 256, kBK = 128;
constexpr int kModeMx = 3;     // MXFP8: E8M0 scales per 32-element block, applied by the scaled MFMA
constexpr int kThreads = 512;
constexpr int kStageA = kBM * kBK;              // 32 KB
constexpr int kStageB = kBN * kBK;              // 32 KB
constexpr int kStageBytes = kStageA + kStageB + 1024 + 1024;   // + sA tile + sB tile (fp32 x 256)

// D = X * Y + Cin for X: 32x64 (lanes index rows), Y: 64x32 (lanes index columns), E4M3.
// Zero scale operands select the unscaled instruction.
__device__ __forceinline__ v16f mfma_32x32x64_e4m3(v8i x, v8i y, v16f c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x, y, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ v8i join(g_u32x4 a, g_u32x4 b) {
  v8i r;
  r[0] = (int)a[0]; r[1] = (int)a[1]; r[2] = (int)a[2]; r[3] = (int)a[3];
  r[4] = (int)b[0]; r[5] = (int)b[1]; r[6] = (int)b[2]; r[7] = (int)b[3];
  return r;
}

// 32-bit LDS byte address of a pointer into shared memory
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

__device__ __forceinline__ void g2lds16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds((glb_void*)g, (lds_void*)lds, 16, 0, 0);
}
__device__ __forceinline__ void g2lds4(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds((glb_void*)g, (lds_void*)lds, 4, 0, 0);
}

// Swizzled position of 16-byte chunk c in a 128-byte LDS row r.  Consecutive row pairs
// share a 256-byte bank line (64 banks x 4 bytes); XOR-ing the chunk with (r >> 1) & 7 spreads
// the 16 rows that one ds_read_b128 quarter-wave touches over all 64 banks.
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 1) & 7); }

// QUANT: the epilogue also writes the 1x128 quantization of the bf16 output (a kernel of its own,
// so that the plain GEMM carries none of it and profiles tell the two apart).
template <int MODE, bool OUT_BF16, bool QUANT>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs p) {
  static_assert(!QUANT || (OUT_BF16 && MODE != kModeMx), "output quantization needs a blockwise bf16 GEMM");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int t = threadIdx.x;
  const int lane = t & 63;
  // wave index as a wave-uniform (scalar) value, so per-wave pointers live in SGPRs
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, h = lane >> 5;
  int tm, tn;
  int split;
  block_of(blockIdx.x, p.tiles_m, p.tiles_n, p.splits, p.group, split, tm, tn);
  const int m0 = tm * kBM, n0 = tn * kBN;
  const int nk = p.K / kBK;                       // slices of the whole contraction
  const int kb_begin = split * p.kb_per_split;    // this block's slice range
  const int kb_end = min(kb_begin + p.kb_per_split, nk);

  // ---- global -> LDS copy plan.  Wave w moves rows 32w .. 32w+31 of the A and B tiles as
  // four 8-row groups; one global_load_lds_dwordx4 moves one group (64 lanes x 16 bytes).
  // The group's first row is wave-uniform (clamped as a whole: M - m0 is a multiple of 128,
  // so a group is either entirely inside or entirely outside the matrix), and each lane
  // adds its own row-in-group and swizzled chunk.
  const int crow = lane >> 3;
  const uint8_t* a_grp[4];
  const uint8_t* b_grp[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r0 = wave * 32 + q * 8;
    a_grp[q] = p.A + (int64_t)min(m0 + r0, p.M - 8) * p.lda;
    b_grp[q] = p.B + (int64_t)min(n0 + r0, p.N - 8) * p.ldb;
  }
  // The lane lands at physical chunk (lane & 7) of row r = 32 wave + 8 q + crow and fetches the
  // logical chunk stored there, swz(r, lane & 7); (r >> 1) & 7 = (4 q + (crow >> 1)) & 7, so
  // even and odd groups q need different lane offsets.
  uint32_t a_off[2], b_off[2];
#pragma unroll
  for (int qp = 0; qp < 2; ++qp) {
    const uint32_t ch = (uint32_t)(swz(qp * 8 + crow, lane & 7) << 4);
    a_off[qp] = (uint32_t)(crow * p.lda) + ch;
    b_off[qp] = (uint32_t)(crow * p.ldb) + ch;
  }
  // scale tiles travel with the operand tiles, so one wait covers a whole slice:
  //   wave 0: sA[kb][m0 .. m0+255] (4 floats per lane);
  //   wave 1: WGRAD sB[kb][n0 .. n0+255]; FWD/DGRAD the two 128-block weight scales
  //           sB[n0/128 + l][kb] (lanes 0 and 1; the other lanes repeat lane 1's address).
  const int s_m = min(m0 + lane * 4, p.M - 4);
  const int s_n = min(n0 + lane * 4, p.N - 4);
  const int64_t s_blk = (int64_t)min((n0 >> 7) + min(lane, 1), (p.N >> 7) - 1) * nk;

  auto issue_scales = [&](int kb, int stage) {
    uint8_t* st = smem + stage * kStageBytes;
    if constexpr (MODE == kModeMx) {
      // E8M0 tiles: [K/128][rows][4] bytes; 256 rows x 4 bytes = 1 KB per operand per slice
      const uint8_t* xa = reinterpret_cast<const uint8_t*>(p.sA);
      const uint8_t* xb = reinterpret_cast<const uint8_t*>(p.sB);
      if (wave == 0) g2lds16(xa + ((int64_t)kb * p.ldsa + s_m) * 4, st + kStageA + kStageB);
      if (wave == 1) g2lds16(xb + ((int64_t)kb * p.N + s_n) * 4, st + kStageA + kStageB + 1024);
      return;
    }
    if (wave == 0) g2lds16(p.sA + (int64_t)kb * p.ldsa + s_m, st + kStageA + kStageB);
    if (wave == 1) {
      if (MODE == 2)
        g2lds16(p.sB + (int64_t)kb * p.N + s_n, st + kStageA + kStageB + 1024);
      else
        g2lds4(p.sB + s_blk + kb, st + kStageA + kStageB + 1024);
    }
  };
  auto issue_slice = [&](int kb, int stage) {
    uint8_t* st = smem + stage * kStageBytes;
    const int64_t ko = (int64_t)kb * kBK;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      g2lds16(a_grp[q] + ko + a_off[q & 1], st + (wave * 32 + q * 8) * kBK);
      g2lds16(b_grp[q] + ko + b_off[q & 1], st + kStageA + (wave * 32 + q * 8) * kBK);
    }
    issue_scales(kb, stage);
  };

  // accumulator of output tile (row group mi, column tile ni) is acc[2 * ni + mi]
  v16f acc[8];
#pragma unroll
  for (int T = 0; T < 8; ++T)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[T][v] = 0.0f;
  v16f zero;
#pragma unroll
  for (int v = 0; v < 16; ++v) zero[v] = 0.0f;

  // fragment reads: lane reads 64 bytes (chunks 4h .. 4h+3) of row r; the swizzle term of
  // every row this lane reads is (l32 >> 1) & 7 (tile row offsets are multiples of 32)
  const int fsw = (l32 >> 1) & 7;
  // Which 16-byte chunks of the slice a lane feeds.  Blockwise modes: chunks 4h .. 4h+3 (any
  // order that A and B share gives the same slice sum).  MX: within one scaled MFMA, the
  // 16-byte groups g = 0, 1 of both lane halves form two 32-element scale blocks, block g taking
  // its scale from lane half g (measured on gfx950).  Lane half h therefore feeds chunks h,
  // h + 4 (first MFMA: MX blocks 0 and 2) and h + 2, h + 6 (second MFMA: MX blocks 1 and 3), so
  // that each hardware block is one MX block and lane half h supplies the scales of MX blocks
  // 2h and 2h + 1, one 16-bit read.
  const int fch[4] = {MODE == kModeMx ? h : 4 * h, MODE == kModeMx ? h + 4 : 4 * h + 1,
                      MODE == kModeMx ? h + 2 : 4 * h + 2, MODE == kModeMx ? h + 6 : 4 * h + 3};
  const int fcol[4] = {(fch[0] ^ fsw) << 4, (fch[1] ^ fsw) << 4, (fch[2] ^ fsw) << 4, (fch[3] ^ fsw) << 4};

  // product of the last tile of a slice, promoted by the next slice's block (WGRAD: together
  // with the column scales of the last column tile)
  v16f pcarry = zero, sbcarry = zero;
  float scp = 0.0f;

  issue_slice(kb_begin, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int kb = kb_begin; kb < kb_end; ++kb) {
    const int stage = (kb - kb_begin) & 1;
    const uint8_t* st = smem + stage * kStageBytes;
    const float* sAs = reinterpret_cast<const float*>(st + kStageA + kStageB);
    const float* sBs = reinterpret_cast<const float*>(st + kStageA + kStageB + 1024);

    // row scales of the lane's two rows; FWD/DGRAD fold in the 128x128 weight-block scale
    // (the wave's 128 columns lie in one block, index wn)
    float sc0 = 0.0f, sc1 = 0.0f;
    if constexpr (MODE != kModeMx) {
      const float sbb = (MODE != 2) ? sBs[wn] : 1.0f;
      sc0 = sAs[wm * 64 + l32] * sbb;
      sc1 = sAs[wm * 64 + 32 + l32] * sbb;
    }

    // LDS byte addresses of this lane's four swizzled 16-byte chunks in its A row and in its B
    // row of the current stage
    const uint32_t sbase = lds_addr(st);
    const uint32_t arow = sbase + (uint32_t)((wm * 64 + l32) * kBK);
    const uint32_t brow = sbase + (uint32_t)(kStageA + (wn * 128 + l32) * kBK);
    // next slice (the last slice re-copies itself into the idle stage, so the block has no
    // branch); its scales are copied here, after this slice's scales were read
    const int kn = kb + 1 < kb_end ? kb + 1 : kb;
    if (kb + 1 < kb_end) issue_scales(kb + 1, stage ^ 1);
    const int64_t ko = (int64_t)kn * kBK;
    const uint32_t m0 = lds_addr(smem + (stage ^ 1) * kStageBytes) + (uint32_t)(wave * 32 * kBK);
    if constexpr (MODE == kModeMx) {
      // the lane's E8M0 pairs: rows wm*64 + mi*32 + l32 of A, wn*128 + ni*32 + l32 of B, MX blocks
      // 2h (first MFMA) and 2h + 1 (second) of the slice (mi, ni offsets are immediates)
      const uint32_t xaj = sbase + (uint32_t)(kStageA + kStageB + (wm * 64 + l32) * 4 + 2 * h);
      const uint32_t xbj = sbase + (uint32_t)(kStageA + kStageB + 1024 + (wn * 128 + l32) * 4 + 2 * h);
      asm volatile(PURO_SLICE_ASM_MXSCALE
                   : "+{v[0:15]}"(acc[0]), "+{v[16:31]}"(acc[1]), "+{v[32:47]}"(acc[2]), "+{v[48:63]}"(acc[3]),
                     "+{v[64:79]}"(acc[4]), "+{v[80:95]}"(acc[5]), "+{v[96:111]}"(acc[6]), "+{v[112:127]}"(acc[7])
                   : [aj0] "v"(arow + fcol[0]), [aj1] "v"(arow + fcol[1]), [aj2] "v"(arow + fcol[2]),
                     [aj3] "v"(arow + fcol[3]), [bj0] "v"(brow + fcol[0]), [bj1] "v"(brow + fcol[1]),
                     [bj2] "v"(brow + fcol[2]), [bj3] "v"(brow + fcol[3]), [xaj] "v"(xaj), [xbj] "v"(xbj),
                     [ga0] "s"(a_grp[0] + ko), [ga1] "s"(a_grp[1] + ko), [ga2] "s"(a_grp[2] + ko),
                     [ga3] "s"(a_grp[3] + ko), [gb0] "s"(b_grp[0] + ko), [gb1] "s"(b_grp[1] + ko),
                     [gb2] "s"(b_grp[2] + ko), [gb3] "s"(b_grp[3] + ko), [oa0] "v"(a_off[0]), [oa1] "v"(a_off[1]),
                     [ob0] "v"(b_off[0]), [ob1] "v"(b_off[1]), [m0] "s"(m0)
                   : PURO_SLICE_ASM_MX_CLOBBERS, "m0", "scc", "memory");
    } else if constexpr (MODE != 2) {
      asm volatile(PURO_SLICE_ASM_ROWSCALE
                   : "+{v[0:15]}"(acc[0]), "+{v[16:31]}"(acc[1]), "+{v[32:47]}"(acc[2]), "+{v[48:63]}"(acc[3]),
                     "+{v[64:79]}"(acc[4]), "+{v[80:95]}"(acc[5]), "+{v[96:111]}"(acc[6]), "+{v[112:127]}"(acc[7]),
                     "+{v[144:159]}"(pcarry)
                   : [aj0] "v"(arow + fcol[0]), [aj1] "v"(arow + fcol[1]), [aj2] "v"(arow + fcol[2]),
                     [aj3] "v"(arow + fcol[3]), [bj0] "v"(brow + fcol[0]), [bj1] "v"(brow + fcol[1]),
                     [bj2] "v"(brow + fcol[2]), [bj3] "v"(brow + fcol[3]), [sc0] "v"(sc0), [sc1] "v"(sc1),
                     [scp] "v"(scp),
                     [ga0] "s"(a_grp[0] + ko), [ga1] "s"(a_grp[1] + ko), [ga2] "s"(a_grp[2] + ko),
                     [ga3] "s"(a_grp[3] + ko), [gb0] "s"(b_grp[0] + ko), [gb1] "s"(b_grp[1] + ko),
                     [gb2] "s"(b_grp[2] + ko), [gb3] "s"(b_grp[3] + ko), [oa0] "v"(a_off[0]), [oa1] "v"(a_off[1]),
                     [ob0] "v"(b_off[0]), [ob1] "v"(b_off[1]), [m0] "s"(m0)
                   : PURO_SLICE_ASM_CLOBBERS, "m0", "scc", "memory");
    } else {
      // the lane's column scales: columns wn*128 + ni*32 + 8g + 4h .. +3 (ni, g immediates)
      const uint32_t sbj = sbase + (uint32_t)(kStageA + kStageB + 1024 + (wn * 128 + 4 * h) * 4);
      asm volatile(PURO_SLICE_ASM_COLSCALE
                   : "+{v[0:15]}"(acc[0]), "+{v[16:31]}"(acc[1]), "+{v[32:47]}"(acc[2]), "+{v[48:63]}"(acc[3]),
                     "+{v[64:79]}"(acc[4]), "+{v[80:95]}"(acc[5]), "+{v[96:111]}"(acc[6]), "+{v[112:127]}"(acc[7]),
                     "+{v[144:159]}"(pcarry), "+{v[208:223]}"(sbcarry)
                   : [aj0] "v"(arow + fcol[0]), [aj1] "v"(arow + fcol[1]), [aj2] "v"(arow + fcol[2]),
                     [aj3] "v"(arow + fcol[3]), [bj0] "v"(brow + fcol[0]), [bj1] "v"(brow + fcol[1]),
                     [bj2] "v"(brow + fcol[2]), [bj3] "v"(brow + fcol[3]), [sa0] "v"(sc0), [sa1] "v"(sc1),
                     [sap] "v"(scp), [sbj] "v"(sbj),
                     [ga0] "s"(a_grp[0] + ko), [ga1] "s"(a_grp[1] + ko), [ga2] "s"(a_grp[2] + ko),
                     [ga3] "s"(a_grp[3] + ko), [gb0] "s"(b_grp[0] + ko), [gb1] "s"(b_grp[1] + ko),
                     [gb2] "s"(b_grp[2] + ko), [gb3] "s"(b_grp[3] + ko), [oa0] "v"(a_off[0]), [oa1] "v"(a_off[1]),
                     [ob0] "v"(b_off[0]), [ob1] "v"(b_off[1]), [m0] "s"(m0)
                   : PURO_SLICE_ASM_COLSCALE_CLOBBERS, "m0", "scc", "memory");
    }
    scp = sc1;  // tile 7's product stays in pcarry until the next block (or the tail)
    // (the block ended with the slice's wait and barrier)
  }

  if constexpr (MODE == kModeMx)
    asm volatile(PURO_SLICE_ASM_MX_TAIL
                 : "+{v[0:15]}"(acc[0]), "+{v[16:31]}"(acc[1]), "+{v[32:47]}"(acc[2]), "+{v[48:63]}"(acc[3]),
                   "+{v[64:79]}"(acc[4]), "+{v[80:95]}"(acc[5]), "+{v[96:111]}"(acc[6]), "+{v[112:127]}"(acc[7]));
  else if constexpr (MODE != 2)
    asm volatile(PURO_SLICE_ASM_ROWSCALE_TAIL : "+{v[112:127]}"(acc[7]) : "{v[144:159]}"(pcarry), [scp] "v"(scp));
  else
    asm volatile(PURO_SLICE_ASM_COLSCALE_TAIL : "+{v[112:127]}"(acc[7]), "+{v[144:159]}"(pcarry)
                 : "{v[208:223]}"(sbcarry), [sap] "v"(scp));

  // ---- epilogue through LDS (free after the loop's last barrier): each wave stages its own
  // output tile, one 32-row half at a time, in a private LDS region with a padded row stride
  // (272 B for bf16, 528 B for fp32: rows land 4 banks apart), then writes whole 256 / 512-
  // byte row segments with 16-byte stores.  The fp32 regions of the 8 waves take exactly the
  // 2 x 66 KB the main loop used.
  const bool rows_ok = m0 + wm * 64 < p.M;
  const bool cols_ok = n0 + wn * 128 < p.N;
  constexpr int kEs = OUT_BF16 ? 2 : 4;                  // output element size
  constexpr int kRow = 128 * kEs + 16;                   // staged row stride (bytes)
  constexpr int kLanesPerRow = 128 * kEs / 16;           // 16 (bf16) or 32 (fp32)
  constexpr int kRowsPerIt = 64 / kLanesPerRow;
  static_assert(8 * 32 * kRow <= 2 * kStageBytes, "epilogue staging exceeds the LDS allocation");
  uint8_t* wbuf = smem + wave * (32 * kRow);
  const int rr = lane / kLanesPerRow, rc = lane % kLanesPerRow;
  // 1x128 output quantization (bf16 output, optional): a wave's 128 columns are one group; the
  // lane holds 64 of its row's values and lane ^ 32 the other 64.  The codes are staged per wave
  // after the C staging area (8 x 32 x 272 + 8 x 32 x 144 bytes <= 2 x 66 KB).
  constexpr int kQRow = 128 + 16;
  static_assert(!QUANT || 8 * 32 * (kRow + kQRow) <= 2 * kStageBytes, "code staging exceeds the LDS allocation");
  uint8_t* qbuf = smem + 8 * 32 * kRow + wave * (32 * kQRow);
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
    [[maybe_unused]] uint32_t am2 = 0;     // packed |bf16| max of this lane's 64 outputs of the row
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint8_t* dst = wbuf + l32 * kRow + (ni * 32 + 8 * g + 4 * h) * kEs;
        if constexpr (OUT_BF16) {
          g_u32x2 o;
          o[0] = bf16x2_rne(acc[2 * ni + mi][4 * g + 0], acc[2 * ni + mi][4 * g + 1]);
          o[1] = bf16x2_rne(acc[2 * ni + mi][4 * g + 2], acc[2 * ni + mi][4 * g + 3]);
          *reinterpret_cast<g_u32x2*>(dst) = o;
          if constexpr (QUANT) am2 = pk_max_u16(am2, pk_max_u16(abs2(o[0]), abs2(o[1])));
        } else {
          const g_f32x4 o = {acc[2 * ni + mi][4 * g + 0], acc[2 * ni + mi][4 * g + 1],
                             acc[2 * ni + mi][4 * g + 2], acc[2 * ni + mi][4 * g + 3]};
          *reinterpret_cast<g_f32x4*>(dst) = o;
        }
      }
    if constexpr (QUANT) {
      // the same numerics as quant_1x128_kernel, applied to the bf16 values just written
      uint32_t am = hmax16(am2);
      am = umax(am, (uint32_t)__shfl_xor((int)am, 32));
      float sc, r;
      tile_scale(am, sc, r);
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const g_u32x2 o = *reinterpret_cast<const g_u32x2*>(wbuf + l32 * kRow + (ni * 32 + 8 * g + 4 * h) * kEs);
          *reinterpret_cast<uint32_t*>(qbuf + l32 * kQRow + ni * 32 + 8 * g + 4 * h) =
              cvt4(bf16_lo(o[0]) * r, bf16_hi(o[0]) * r, bf16_lo(o[1]) * r, bf16_hi(o[1]) * r);
        }
      if (h == 0 && rows_ok && cols_ok)
        p.qs[(int64_t)((n0 >> 7) + wn) * p.ldqs + m0 + wm * 64 + mi * 32 + l32] = sc;
    }
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    if (QUANT && rows_ok && cols_ok) {
      uint8_t* qrow = p.q + (int64_t)(m0 + wm * 64 + mi * 32) * p.ldq + n0 + wn * 128;
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int r = it * 8 + (lane >> 3), part = lane & 7;
        *reinterpret_cast<g_u32x4*>(qrow + (int64_t)r * p.ldq + part * 16) =
            *reinterpret_cast<const g_u32x4*>(qbuf + r * kQRow + part * 16);
      }
    }
    if (rows_ok && cols_ok) {
      uint8_t* cbase = static_cast<uint8_t*>(p.C) +
                       ((int64_t)split * p.split_stride + (int64_t)(m0 + wm * 64 + mi * 32) * p.ldc + n0 + wn * 128) * kEs;
#pragma unroll
      for (int it = 0; it < 32 / kRowsPerIt; ++it) {
        const int r = it * kRowsPerIt + rr;
        g_u32x4 v = *reinterpret_cast<const g_u32x4*>(wbuf + r * kRow + rc * 16);
        g_u32x4* cp = reinterpret_cast<g_u32x4*>(cbase + (int64_t)r * p.ldc * kEs + rc * 16);
        if (!OUT_BF16 && p.accumulate) {
          const g_f32x4 sum = __builtin_bit_cast(g_f32x4, v) + __builtin_bit_cast(g_f32x4, *cp);
          v = __builtin_bit_cast(g_u32x4, sum);
        }
        *cp = v;
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
  }
}

// Zero-fill of C for an empty contraction (K == 0): the exact result is 0.
__global__ __launch_bounds__(256) void zero_fill_kernel(void* __restrict__ C, int64_t M, int64_t rowbytes,
                                                        int64_t ldbytes) {
  const int64_t words = rowbytes >> 2;
  for (int64_t i = blockIdx.y; i < M; i += gridDim.y)
    for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < words; w += (int64_t)gridDim.x * blockDim.x)
      reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(C) + i * ldbytes)[w] = 0u;
}

// Sum of the fp32 partials of a split contraction, in split order (deterministic), written as
// bf16 (round to nearest even) or fp32 (optionally added to C).  4 consecutive columns per thread.
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void split_reduce_kernel(const float* __restrict__ part, int splits,
                                                           int64_t split_stride, int M, int N,
                                                           void* __restrict__ C, int64_t ldc, int accumulate) {
  const int64_t n4 = N >> 2;
  const int64_t total = (int64_t)M * n4;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = e / n4, j = (e - i * n4) * 4;
    g_f32x4 acc = *reinterpret_cast<const g_f32x4*>(part + i * N + j);
    for (int sp = 1; sp < splits; ++sp) acc += *reinterpret_cast<const g_f32x4*>(part + sp * split_stride + i * N + j);
    if (OUT_BF16) {
      g_u32x2 o;
      o[0] = bf16x2_rne(acc[0], acc[1]);
      o[1] = bf16x2_rne(acc[2], acc[3]);
      *reinterpret_cast<g_u32x2*>(static_cast<uint16_t*>(C) + i * ldc + j) = o;
    } else {
      g_f32x4* cp = reinterpret_cast<g_f32x4*>(static_cast<float*>(C) + i * ldc + j);
      if (accumulate) acc = acc + *cp;   // after the in-order sum: the same single add as unsplit
      *cp = acc;
    }
  }
}

// Contraction split for a problem: the smallest estimated time among 1, 2, 4 and 8 splits,
// modelling whole waves of 256 workgroups (one per CU), ~3 slices of fixed cost per
// workgroup, and the partials' HBM round trip (~1 slice time per 10 MB).
static int choose_splits(int64_t M, int64_t N, int64_t K) {
  const int64_t tiles = ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
  const int64_t nk = K / kBK;
  int best = 1;
  double best_t = 1e300;
  for (int sp = 1; sp <= 8; sp *= 2) {
    if (nk / sp < 8) break;
    const double waves = (double)((tiles * sp + 255) / 256);
    const double per_block = (double)((nk + sp - 1) / sp) + 3.0;
    const double reduce = sp > 1 ? (double)(sp + 1) * M * N * 4 / 10.0e6 : 0.0;
    const double t = waves * per_block + reduce;
    if (t < best_t * 0.97) {
      best_t = t;
      best = sp;
    }
  }
  return best;
}

template <int MODE, bool BF16, bool QUANT = false>
static hipError_t launch_one(const GemmArgs& a, hipStream_t st) {
  const int smem = 2 * kStageBytes;
  // The dynamic-LDS limit is a per-device attribute of the kernel: set it once per device the
  // caller launches on (threads that race here all set the same value).
  constexpr int kMaxDevices = 64;
  static std::atomic<bool> attr_set[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool known = dev >= 0 && dev < kMaxDevices;
  if (!known || !attr_set[dev].load(std::memory_order_acquire)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_kernel<MODE, BF16, QUANT>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, smem);
    if (e != hipSuccess) return e;
    if (known) attr_set[dev].store(true, std::memory_order_release);
  }
  hipLaunchKernelGGL((gemm_kernel<MODE, BF16, QUANT>), dim3(a.tiles_m * a.tiles_n * a.splits), dim3(kThreads), smem, st, a);
  return hipGetLastError();
}

// FWD and DGRAD (without the fused output quantization) run the four-wave kernel of gemm_w4.hip
// wherever its 32-bit operand offsets reach (w4_supported), the eight-wave kernel elsewhere.
#ifndef PURO_GEMM_W4
#define PURO_GEMM_W4 1
#endif
constexpr bool kUseW4 = PURO_GEMM_W4 != 0;

// Tile rows per group (see block_of).  The A rows of a group take group x 256 x K bytes of
// the XCD's 4 MB L2.  Up to K = 2048, 4 rows (2 MB) stay resident from one wave of tiles to
// the next while the B columns stream past, and 8 rows (4 MB) would not (measured on MI355X at
// 16384 tokens: 16384 x 12288 x 2048 FWD gains 13% with 4 rows).  Beyond that no group's rows
// survive a wave, and what counts is how many operand panels (tile rows plus tile columns) the
// up to 32 workgroups an XCD runs at once touch: 8 rows, unless 4 touch fewer (a 192-workgroup
// grid's 24 per XCD: 4 rows x 6 columns against 8 x 3).
static int choose_group(int64_t M, int64_t N, int64_t K, int splits) {
  if (K <= 2048) return 4;
  const int64_t tm = (M + kBM - 1) / kBM, tn = (N + kBN - 1) / kBN;
  const int64_t run = std::max<int64_t>(1, std::min<int64_t>(32, tm * tn * splits / 8));
  auto panels = [&](int64_t g) {
    const int64_t rows = std::min(g, tm);
    return rows + std::min(tn, (run + rows - 1) / rows);
  };
  return panels(4) < panels(8) ? 4 : 8;
}

// One GEMM launch (and its split-K reduce) over M rows of A and C; the slices of sA are ldsa
// apart (ldsa >= M).
static hipError_t launch_rows(int mode, int64_t M, int64_t N, int64_t K, int splits, const uint8_t* A,
                              int64_t lda, const float* sA, int64_t ldsa, const uint8_t* B, int64_t ldb,
                              const float* sB, void* C, int64_t ldc, bool out_bf16, bool accumulate, uint8_t* q,
                              int64_t ldq, float* qs, int64_t ldqs, void* workspace, size_t workspace_bytes,
                              hipStream_t st) {
  GemmArgs a;
  a.M = (int)M; a.N = (int)N; a.K = (int)K;
  a.tiles_m = (int)((M + kBM - 1) / kBM);
  a.tiles_n = (int)((N + kBN - 1) / kBN);
  if ((int64_t)a.tiles_m * a.tiles_n > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  a.A = A; a.lda = lda; a.sA = sA; a.ldsa = ldsa; a.B = B; a.ldb = ldb; a.sB = sB; a.C = C; a.ldc = ldc;
  a.accumulate = 0;
  a.q = nullptr; a.ldq = 0; a.qs = nullptr; a.ldqs = 0;
  a.splits = splits;
  a.group = choose_group(M, N, K, splits);
  a.kb_per_split = (int)((K / kBK + a.splits - 1) / a.splits);
  a.split_stride = 0;
  if (a.splits > 1) {
    // partial sums (fp32, [split][M][N]) in the caller's workspace, then one reduction
    if (workspace == nullptr || workspace_bytes < (size_t)a.splits * (size_t)M * (size_t)N * 4) return hipErrorInvalidValue;
    a.C = workspace;
    a.ldc = N;
    a.split_stride = M * N;
    hipError_t e;
    const bool w4 = kUseW4 && w4_supported(a);
    switch (mode) {
      case 0: e = w4 ? launch_w4(a, false, st) : launch_one<0, false>(a, st); break;
      case 1: e = w4 ? launch_w4(a, false, st) : launch_one<1, false>(a, st); break;
      case 2: e = launch_one<2, false>(a, st); break;
      default: e = kUseW4 && w4mx_supported(a) ? launch_w4mx(a, false, st) : launch_one<kModeMx, false>(a, st); break;
    }
    if (e != hipSuccess) return e;
    const int64_t work = M * (N / 4);
    const int64_t blocks = std::min<int64_t>((work + 255) / 256, 4096);
    if (out_bf16) {
      hipLaunchKernelGGL(split_reduce_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, st,
                         static_cast<const float*>(workspace), a.splits, a.split_stride, (int)M, (int)N, C, ldc, 0);
      if (q != nullptr) {   // quantize the reduced bf16 output: the same bytes as the fused epilogue
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        return launch_quant_1x128(C, M, N, ldc, q, ldq, qs, st, ldqs);
      }
    }
    else
      hipLaunchKernelGGL(split_reduce_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, st,
                         static_cast<const float*>(workspace), a.splits, a.split_stride, (int)M, (int)N, C, ldc,
                         accumulate ? 1 : 0);
    return hipGetLastError();
  }
  a.accumulate = accumulate ? 1 : 0;
  a.q = q; a.ldq = ldq; a.qs = qs; a.ldqs = ldqs;
  if (q != nullptr) {
    if (kUseW4 && (mode == 0 || mode == 1) && w4_supported(a)) return launch_w4(a, true, st);
    switch (mode) {
      case 0: return launch_one<0, true, true>(a, st);
      case 1: return launch_one<1, true, true>(a, st);
      case 2: return launch_one<2, true, true>(a, st);
      default: return hipErrorInvalidValue;
    }
  }
  if (kUseW4 && (mode == 0 || mode == 1) && w4_supported(a)) return launch_w4(a, out_bf16, st);
  if (kUseW4 && mode == kModeMx && !accumulate && w4mx_supported(a)) return launch_w4mx(a, out_bf16, st);
  switch (mode * 2 + (out_bf16 ? 1 : 0)) {
    case 0: return launch_one<0, false>(a, st);
    case 1: return launch_one<0, true>(a, st);
    case 2: return launch_one<1, false>(a, st);
    case 3: return launch_one<1, true>(a, st);
    case 4: return launch_one<2, false>(a, st);
    case 5: return launch_one<2, true>(a, st);
    case 6: return launch_one<kModeMx, false>(a, st);
    default: return launch_one<kModeMx, true>(a, st);
  }
}

// Rows of a leading part that runs without a contraction split, when the whole problem would be
// split only to fill its last, partial wave of tiles: the whole waves first (as whole tile rows),
// then the remaining rows with a split of their own.  Only the remaining rows' partials then go
// through the workspace and the reduce (measured on MI355X, WGRAD 12288 x 2048 x 16384: 487 us as
// one split launch, 432 us as 8192 unsplit rows + 4096 split rows).  0 = no such part.
static int64_t leading_rows(int64_t M, int64_t N, int64_t K) {
  constexpr int64_t kWave = 256;                 // workgroups per wave (one per CU), as choose_splits
  const int64_t tn = (N + kBN - 1) / kBN, tm = (M + kBM - 1) / kBM;
  if (kWave % tn != 0) return 0;                 // a wave must be whole tile rows
  const int64_t rows_per_wave = kWave / tn;
  const int64_t waves = tm / rows_per_wave;
  if (waves == 0 || waves * rows_per_wave == tm) return 0;
  if (choose_splits(M, N, K) == 1) return 0;
  const int64_t M1 = waves * rows_per_wave * kBM;
  if (choose_splits(M - M1, N, K) == 1) return 0;
  return M1;
}

int gemm_parts(int64_t M, int64_t N, int64_t K, GemmPart parts[2]) {
  const int64_t M1 = leading_rows(M, N, K);
  if (M1 > 0) {
    parts[0] = GemmPart{0, M1, 1};
    parts[1] = GemmPart{M1, M - M1, choose_splits(M - M1, N, K)};
    return 2;
  }
  parts[0] = GemmPart{0, M, choose_splits(M, N, K)};
  return 1;
}

size_t part_workspace(const GemmPart& p, int64_t N) {
  return p.splits > 1 ? (size_t)p.splits * (size_t)p.rows * (size_t)N * 4 : 0;
}

// Split-K partials of the allocation-free entry point.  Uninitialized device memory, loaded with the
// code object on each device the library runs on and kept until the process ends.  In host code
// this name is not a device address: kernels get the address scratch_buffer looked up.
static __device__ __attribute__((aligned(256))) uint8_t scratch[kScratchBytes];

hipError_t scratch_buffer(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> addr[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    // the device's own copy of the array (threads racing here all find the same address)
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

// The workspace of a call (puro_fp8_gemm, puro_fp8_gemm_accumulate and puro_fp8_gemm_quant follow
// the same plan): its largest part.
size_t gemm_workspace_bytes(int, int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  GemmPart parts[2];
  const int n = gemm_parts(M, N, K, parts);
  size_t need = 0;
  for (int i = 0; i < n; ++i) need = std::max(need, part_workspace(parts[i], N));
  return need;
}

hipError_t launch_gemm(int mode, int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                       const float* sA, const uint8_t* B, int64_t ldb, const float* sB, void* C,
                       int64_t ldc, bool out_bf16, bool accumulate, uint8_t* q, int64_t ldq, float* qs,
                       void* workspace, size_t workspace_bytes, hipStream_t st) {
  if (accumulate && out_bf16) return hipErrorInvalidValue;
  if (q != nullptr && !out_bf16) return hipErrorInvalidValue;
  if (K == 0) {
    if (accumulate) return hipSuccess;   // C + 0
    if (q != nullptr) {
      const int64_t gy = M < 65535 ? M : 65535;
      hipLaunchKernelGGL(zero_fill_kernel, dim3(8, (unsigned)gy), dim3(256), 0, st, C, M, N * 2, ldc * 2);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      return launch_quant_1x128(C, M, N, ldc, q, ldq, qs, st);
    }

    const int64_t es = out_bf16 ? 2 : 4;
    const int64_t gy = M < 65535 ? M : 65535;
    hipLaunchKernelGGL(zero_fill_kernel, dim3(8, (unsigned)gy), dim3(256), 0, st, C, M, N * es, ldc * es);
    return hipGetLastError();
  }
  GemmPart parts[2];
  const int n = gemm_parts(M, N, K, parts);
  // every part's workspace is checked before the first launch: a failed call writes nothing
  for (int i = 0; i < n; ++i) {
    const size_t need = part_workspace(parts[i], N);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return hipErrorInvalidValue;
  }
  const int64_t es = out_bf16 ? 2 : 4;
  for (int i = 0; i < n; ++i) {
    const GemmPart& pt = parts[i];
    // sA (and the MX E8M0 tiles, 4 bytes per row) and the output scales of row r start r elements in
    const hipError_t e =
        launch_rows(mode, pt.rows, N, K, pt.splits, A + pt.row0 * lda, lda, sA + pt.row0, M, B, ldb, sB,
                    static_cast<uint8_t*>(C) + pt.row0 * ldc * es, ldc, out_bf16, accumulate,
                    q ? q + pt.row0 * ldq : nullptr, ldq, q ? qs + pt.row0 : nullptr, M, workspace,
                    workspace_bytes, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace puro

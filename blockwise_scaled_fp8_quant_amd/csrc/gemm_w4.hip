// gfx950 blockwise-scaled FP8 GEMM, four-wave form (FWD and DGRAD: one 128x128 weight-block scale per
// 128 columns, so every lane's promotion scale is one value per row group and slice).
//
//   C[i,j] = sum_kb  sA(i,kb) * sB(j/128,kb) * P_kb[i,j],   P_kb[i,j] = sum_{k in slice kb} A[i,k] B[j,k]
//
// The FP8 matrix cores form each 128-deep slice product P_kb (v_mfma_f32_16x16x128_f8f6f4, E4M3 x
// E4M3 -> fp32) and the vector ALUs add it, multiplied by the slice's two scales, into a separate fp32
// accumulator (the fine-grained scheme of the ModelScope write-up on Puro-2B, section 精度).
//
// One workgroup = 4 waves, one per SIMD, owns a 256x256 output tile; wave w (wm = w / 2, wn = w % 2)
// owns the 128x128 quadrant at rows 128 wm, columns 128 wn.  At one wave per SIMD a wave has 256
// VGPRs and 256 AGPRs: the operand fragments of a slice sit in AGPRs (the MFMA reads them there),
// 7/8 of the accumulator in VGPRs and its last column group in AGPRs.  Each slice a wave reads
// 128 + 128 rows of 128 bytes from LDS for 2 * 128 * 128 * 128 flops: a third less LDS read traffic
// per flop than two waves per SIMD with 64x128 tiles.  The slice's instruction sequence is
// generated (gen_w4_asm.py -> gemm_w4_asm.inc; register map and schedule are described there);
// this file sets up its operands, runs the K loop over it and writes the tile out.
//
//  * K loop over 128-deep slices, double-buffered in LDS: while one stage is multiplied, the next
//    slice's A and B rows (256 x 128 bytes each) and scales are copied into the other with
//    buffer_load ... lds (no VGPR round trip).  The buffer resources span the tile's valid rows, so
//    rows past M or N read as zero (half-filled edge tiles need no clamping).
//  * Tiles are visited in the XCD-aware order of block_of (gemm_args.hpp).  Each wave also pulls
//    the slice after next into L2, one dword per row, asking for each line once per XCD (pf_row).
//  * The epilogue stages each wave's quadrant through LDS (bf16: all 128 rows at once; fp32, and
//    bf16 with the fused output quantization: 64 rows at a time) and writes whole row segments
//    with 16-byte stores.
//  * Optionally (QUANT, FWD / DGRAD with bf16 output) the epilogue also writes the 1x128
//    quantization of C along N: a wave's 128 columns are one group, held by the 4 lanes that share
//    a row, and the quantizer's numerics are applied to the bf16 values it writes.
#include <hip/hip_runtime.h>

#include <atomic>

#include "codec.hpp"
#include "gemm_args.hpp"
#include "gemm_w4_asm.inc"
#include "gemm_w4mx_asm.inc"
#include "internal.hpp"

namespace puro {

namespace {

typedef int w4_v4i __attribute__((ext_vector_type(4)));
typedef int w4_v8i __attribute__((ext_vector_type(8)));
typedef float w4_v2f __attribute__((ext_vector_type(2)));
typedef float w4_v4f __attribute__((ext_vector_type(4)));
typedef float w4_v16f __attribute__((ext_vector_type(16)));

constexpr int kW4Threads = 256;
// 2 stages x (A 32 KB + B 32 KB), 2 stages x 2 KB of scales, 256 bytes that the L2 prefetches land in
constexpr int kW4Lds = 131072 + 2 * 2048 + 256;
// the bf16 epilogue stages 4 waves x 128 rows x 272 bytes, a little more than the K loop uses
constexpr int kW4Smem = 4 * 128 * 272 > kW4Lds ? 4 * 128 * 272 : kW4Lds;
constexpr uint32_t kRsrcWord3 = 0x00020000u; // raw buffer, 32-bit data format (gfx9 family)

// Buffer resource of `bytes` bytes at `base` (stride 0: a plain byte range; reads past it return 0).
__device__ __forceinline__ w4_v4i rsrc(const void* base, int64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint64_t n = bytes < 0 ? 0 : (bytes > 0xFFFFFFFFll ? 0xFFFFFFFFull : (uint64_t)bytes);
  w4_v4i r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)((a >> 32) & 0xFFFFu));
  r[2] = __builtin_amdgcn_readfirstlane((int)(uint32_t)n);
  r[3] = (int)kRsrcWord3;
  return r;
}

}  // namespace


// ---- epilogue of both four-wave kernels: `val(mi, ni, r)` is element r (row 16 mi + lane % 16,
// column 16 ni + 4 (lane / 16) + r of the wave's quadrant) of the finished accumulator.
template <bool OUT_BF16, bool QUANT, typename Val>
__device__ __forceinline__ void w4_epilogue(const GemmArgs& p, uint8_t* smem, int wave, int lane, int m0, int n0,
                                            int split, Val val) {
  const int wm = wave >> 1, wn = wave & 1;
  const int l16 = lane & 15, g = lane >> 4;
  // Each wave stages its quadrant in its own LDS region (bf16: all 128 rows; fp32, and bf16 with the
  // output quantization: 64 rows at a time), then writes whole row segments with 16-byte stores,
  // eight rows' reads in flight at a time.  Row strides of 272 / 528 bytes put consecutive rows 4 banks apart: the 32 lanes of a
  // half-wave write 16 rows x 16 bytes (bf16) and hit 64 different banks, and the 16 lanes of a
  // 16-byte read of one row do too.  The last slice block ended with a barrier, so LDS is free; the
  // stores are not waited for (only the LDS reads).
  constexpr int kEs = OUT_BF16 ? 2 : 4;
  constexpr int kRow = 128 * kEs + 16;
  constexpr int kStaged = OUT_BF16 && !QUANT ? 128 : 64; // rows staged per pass
  constexpr int kLanesPerRow = 128 * kEs / 16;           // 16 (bf16) or 32 (fp32)
  constexpr int kRowsPerIt = 64 / kLanesPerRow;          // rows one 16-byte store instruction covers
  constexpr int kBatch = 8;
  static_assert(4 * kStaged * kRow <= kW4Smem, "epilogue staging exceeds the LDS allocation");
  uint8_t* wbuf = smem + wave * (kStaged * kRow);
  // QUANT: the codes of the staged rows, 128 bytes per row at a 144-byte stride (a row of 36 dwords:
  // the 16 rows x 4 lanes of one code write hit 64 different banks), behind the 4 waves' C staging
  constexpr int kQRow = 144;
  static_assert(!QUANT || 4 * kStaged * (kRow + kQRow) <= kW4Smem, "code staging exceeds the LDS allocation");
  uint8_t* qbuf = smem + 4 * kStaged * kRow + wave * (kStaged * kQRow);
  const bool cols_ok = n0 + 128 * wn < p.N;
  const int rr = lane / kLanesPerRow, rc = lane % kLanesPerRow;
#pragma unroll
  for (int h = 0; h < 128 / kStaged; ++h) {
    constexpr int kGroups = kStaged / 16;                // row groups per pass
#pragma unroll
    for (int mi = kGroups * h; mi < kGroups * h + kGroups; ++mi) {
#pragma unroll
      for (int ni = 0; ni < 8; ++ni) {
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = val(mi, ni, r);
        uint8_t* dst = wbuf + (16 * (mi - kGroups * h) + l16) * kRow + (16 * ni + 4 * g) * kEs;
        if constexpr (OUT_BF16) {
          g_u32x2 o;
          o[0] = bf16x2_rne(v[0], v[1]);
          o[1] = bf16x2_rne(v[2], v[3]);
          *reinterpret_cast<g_u32x2*>(dst) = o;
        } else {
          const g_f32x4 o = {v[0], v[1], v[2], v[3]};
          *reinterpret_cast<g_f32x4*>(dst) = o;
        }
      }
      if constexpr (QUANT) {
        // the row's 1x128 group: this lane's 32 bf16 values (columns 16 ni + 4 g .. +3), then the
        // other three lanes of the row (lanes l16 + 16 g); the same numerics as quant_1x128_kernel
        uint32_t am2 = 0;
        g_u32x2 o[8];
#pragma unroll
        for (int ni = 0; ni < 8; ++ni) {
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = val(mi, ni, r);
          o[ni][0] = bf16x2_rne(v[0], v[1]);
          o[ni][1] = bf16x2_rne(v[2], v[3]);
          am2 = pk_max_u16(am2, pk_max_u16(abs2(o[ni][0]), abs2(o[ni][1])));
        }
        uint32_t am = hmax16(am2);
        am = umax(am, (uint32_t)__shfl_xor((int)am, 16));
        am = umax(am, (uint32_t)__shfl_xor((int)am, 32));
        float sc, r;
        tile_scale(am, sc, r);
        const int srow = 16 * (mi - kGroups * h) + l16;           // row within the staged rows
#pragma unroll
        for (int ni = 0; ni < 8; ++ni)
          *reinterpret_cast<uint32_t*>(qbuf + srow * kQRow + 16 * ni + 4 * g) =
              cvt4(bf16_lo(o[ni][0]) * r, bf16_hi(o[ni][0]) * r, bf16_lo(o[ni][1]) * r, bf16_hi(o[ni][1]) * r);
        const int row = m0 + 128 * wm + 16 * mi + l16;
        if (g == 0 && row < p.M && cols_ok) p.qs[(int64_t)((n0 >> 7) + wn) * p.ldqs + row] = sc;
      }
    }
    // the wave reads back its own rows: wait for its LDS writes only
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();
    const int row0 = m0 + 128 * wm + kStaged * h;
    if (row0 < p.M && cols_ok) {
      uint8_t* cbase = static_cast<uint8_t*>(p.C) +
                       ((int64_t)split * p.split_stride + (int64_t)row0 * p.ldc + n0 + 128 * wn) * kEs;
#pragma unroll
      for (int it0 = 0; it0 < kStaged / kRowsPerIt; it0 += kBatch) {
        g_u32x4 v[kBatch];
#pragma unroll
        for (int b = 0; b < kBatch; ++b)
          v[b] = *reinterpret_cast<const g_u32x4*>(wbuf + ((it0 + b) * kRowsPerIt + rr) * kRow + rc * 16);
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
          const int r = (it0 + b) * kRowsPerIt + rr;
          g_u32x4* cp = reinterpret_cast<g_u32x4*>(cbase + (int64_t)r * p.ldc * kEs + rc * 16);
          g_u32x4 o = v[b];
          if (!OUT_BF16 && p.accumulate) {
            const g_f32x4 sum = __builtin_bit_cast(g_f32x4, o) + __builtin_bit_cast(g_f32x4, *cp);
            o = __builtin_bit_cast(g_u32x4, sum);
          }
          *cp = o;
        }
      }
      if constexpr (QUANT) {
        // the staged codes: 8 lanes x 16 bytes per 128-byte row, 8 rows per store instruction
        uint8_t* qrow = p.q + (int64_t)row0 * p.ldq + n0 + 128 * wn;
#pragma unroll
        for (int it = 0; it < kStaged / 8; ++it) {
          const int r = 8 * it + (lane >> 3), part = lane & 7;
          *reinterpret_cast<g_u32x4*>(qrow + (int64_t)r * p.ldq + part * 16) =
              *reinterpret_cast<const g_u32x4*>(qbuf + r * kQRow + part * 16);
        }
      }
    }
    if (h + 1 < 128 / kStaged) {
      // the next pass overwrites the staging area: this pass's reads must have returned
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_wave_barrier();
    }
  }
}

template <bool OUT_BF16, bool QUANT>
__global__ __launch_bounds__(kW4Threads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_w4_kernel(GemmArgs p) {
  static_assert(!QUANT || OUT_BF16, "the fused output quantization needs the bf16 output");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  int tm, tn;
  int split;
  block_of(blockIdx.x, p.tiles_m, p.tiles_n, p.splits, p.group, split, tm, tn);
  const int m0 = tm * 256, n0 = tn * 256;
  const int nk = p.K / 128;
  const int kb_begin = split * p.kb_per_split;
  const int kb_end = min(kb_begin + p.kb_per_split, nk);

  // ---- copy operands (see gen_w4_asm.py): buffer resources over the tile's valid rows
  const w4_v4i rA = rsrc(p.A + (int64_t)m0 * p.lda, (int64_t)min(256, p.M - m0) * p.lda);
  const w4_v4i rB = rsrc(p.B + (int64_t)n0 * p.ldb, (int64_t)min(256, p.N - n0) * p.ldb);
  const w4_v4i rS = rsrc(p.sA + m0, ((int64_t)nk * p.ldsa - m0) * 4);
  const w4_v4i rW = rsrc(p.sB + (int64_t)(n0 >> 7) * nk, (int64_t)((p.N >> 7) - (n0 >> 7)) * nk * 4);
  w4_v8i qa, qb;                                   // the wave's 8-row copy groups
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    qa[q] = __builtin_amdgcn_readfirstlane((int)(uint32_t)((64 * wave + 8 * q) * p.lda));
    qb[q] = __builtin_amdgcn_readfirstlane((int)(uint32_t)((64 * wave + 8 * q) * p.ldb));
  }
  // the lane lands at physical chunk (lane & 7) of row r = 64 wave + 8 q + (lane >> 3) and fetches
  // the logical chunk stored there; (r >> 1) & 7 = ((lane >> 4) + 4 q) & 7, so odd groups flip bit 2
  const int crow = lane >> 3, pch = lane & 7;
  const uint32_t k0 = (uint32_t)kb_begin * 128u;
  uint32_t oa0 = (uint32_t)(crow * p.lda) + (uint32_t)((pch ^ (crow >> 1)) << 4) + k0;
  uint32_t oa1 = (uint32_t)(crow * p.lda) + (uint32_t)((pch ^ (crow >> 1) ^ 4) << 4) + k0;
  uint32_t ob0 = (uint32_t)(crow * p.ldb) + (uint32_t)((pch ^ (crow >> 1)) << 4) + k0;
  uint32_t ob1 = (uint32_t)(crow * p.ldb) + (uint32_t)((pch ^ (crow >> 1) ^ 4) << 4) + k0;
  const uint32_t osa = (uint32_t)lane * 4u;
  // prefetch offsets, two slices ahead of the one being copied (the prologue prefetches the second
  // slice): a row of the wave's 64 (its base row is in qa[0] / qb[0]), the one row of each run of
  // lanes that this tile fetches for the resident tiles sharing the panel (pf_row)
  uint32_t pfa = (uint32_t)(pf_row(lane, tn, pf_share_a(p)) * p.lda) + k0 + 128u;
  uint32_t pfb = (uint32_t)(pf_row(lane, tm, pf_share_b(p)) * p.ldb) + k0 + 128u;
  int ssp;                                         // row-scale offset of the prefetched slice
  int ssa = __builtin_amdgcn_readfirstlane((int)(((int64_t)kb_begin * p.ldsa + 64 * wave) * 4));
  int ssw = __builtin_amdgcn_readfirstlane((wn * nk + kb_begin) * 4);
  const int sstep = __builtin_amdgcn_readfirstlane((int)(p.ldsa * 4));
  const int mw = wave * 8192, ms = 131072 + 256 * wave;

  // ---- fragment read addresses (stage 0): the lane's two 16-byte chunks of its row, g and g + 4 (any
  // assignment that A and B share gives the same slice sum; this one, the MXFP8 kernel's, keeps the
  // reads off each other's banks); every row a lane reads has the swizzle term (lane & 15) >> 1 (row
  // offsets are multiples of 16)
  const int l16 = lane & 15, g = lane >> 4, sw = l16 >> 1;
  const uint32_t c0 = (uint32_t)((g ^ sw) << 4), c1 = (uint32_t)(((g + 4) ^ sw) << 4);
  const uint32_t aj0 = (uint32_t)((128 * wm + l16) * 128) + c0, aj1 = (uint32_t)((128 * wm + l16) * 128) + c1;
  const uint32_t bj0 = 65536u + (uint32_t)((128 * wn + l16) * 128) + c0;
  const uint32_t bj1 = 65536u + (uint32_t)((128 * wn + l16) * 128) + c1;
  const uint32_t sj = 131072u + 4u * (uint32_t)(128 * wm + l16);
  const uint32_t swj = 131072u + 1024u + 256u * (uint32_t)wave;

  // accumulators, products, scales and temporaries: set to zero inside the K loop's asm while the
  // first slice's copies are in flight.  They are early-clobber outputs: written while the inputs
  // are still being read, so they never share a register with an input.
  w4_v16f acc[14];
  w4_v4f agp[8];                 // tiles (mi, 7): as 4-register operands
  w4_v4f p0, p1, p2, tmp;
  w4_v2f sc;

#define PURO_W4_OUTS                                                                                         \
  "=&{v[0:15]}"(acc[0]), "=&{v[16:31]}"(acc[1]), "=&{v[32:47]}"(acc[2]), "=&{v[48:63]}"(acc[3]),             \
      "=&{v[64:79]}"(acc[4]), "=&{v[80:95]}"(acc[5]), "=&{v[96:111]}"(acc[6]), "=&{v[112:127]}"(acc[7]),     \
      "=&{v[128:143]}"(acc[8]), "=&{v[144:159]}"(acc[9]), "=&{v[160:175]}"(acc[10]),                         \
      "=&{v[176:191]}"(acc[11]), "=&{v[192:207]}"(acc[12]), "=&{v[208:223]}"(acc[13]),                       \
      "=&{a[0:3]}"(agp[0]), "=&{a[4:7]}"(agp[1]), "=&{a[8:11]}"(agp[2]), "=&{a[12:15]}"(agp[3]),             \
      "=&{a[16:19]}"(agp[4]), "=&{a[20:23]}"(agp[5]), "=&{a[24:27]}"(agp[6]), "=&{a[28:31]}"(agp[7]),        \
      "=&{v[224:227]}"(p0), "=&{v[228:231]}"(p1), "=&{v[232:235]}"(p2), "=&{v[236:237]}"(sc),                \
      "=&{v[238:241]}"(tmp), "+{v243}"(oa0), "+{v244}"(oa1), "+{v245}"(ob0), "+{v246}"(ob1), "+{v247}"(pfa), \
      "+{v248}"(pfb), [ssa] "+s"(ssa), [ssw] "+s"(ssw), [ssp] "=&s"(ssp), [pairs] "+s"(pairs)
#define PURO_W4_INS                                                                                         \
  [aj0] "v"(aj0), [aj1] "v"(aj1), [bj0] "v"(bj0), [bj1] "v"(bj1), [sj] "v"(sj), [swj] "v"(swj),             \
      [osa] "v"(osa), [rA] "s"(rA), [rB] "s"(rB), [rS] "s"(rS), [rW] "s"(rW), [qa] "{s[64:71]}"(qa),        \
      [qb] "{s[72:79]}"(qb), [sstep] "s"(sstep), [mw] "s"(mw), [ms] "s"(ms), [rem] "s"(rem)
#define PURO_W4_CLOB PURO_W4_CLOBBERS, "v242", "m0", "scc", "memory"

  // slices kb_begin .. kb_end - 1 (at least one): `pairs` stage-0 / stage-1 pairs that copy the
  // slice after them, then the last `rem` (1 or 2) slices
  const int n = kb_end - kb_begin;
  int pairs = __builtin_amdgcn_readfirstlane((n - 1) / 2);
  const int rem = __builtin_amdgcn_readfirstlane(n - 2 * ((n - 1) / 2));
  asm volatile(PURO_W4_MAINLOOP : PURO_W4_OUTS : PURO_W4_INS : PURO_W4_CLOB);
  (void)ssp;
#undef PURO_W4_OUTS
#undef PURO_W4_INS
#undef PURO_W4_CLOB

  w4_epilogue<OUT_BF16, QUANT>(p, smem, wave, lane, m0, n0, split,
                               [&](int mi, int ni, int r) { return ni < 7 ? acc[(7 * mi + ni) >> 2][4 * ((7 * mi + ni) & 3) + r] : agp[mi][r]; });
}

// MXFP8 GEMM in the four-wave form: the same tiles, copies, L2 prefetch and epilogue, with the
// scaled MFMA applying the E8M0 block scales of both operands (gen_w4mx_asm.py) and the
// accumulators in AGPRs.  Scales: A [K/128][M][4] bytes (slices ldsa rows apart), B [K/128][N][4].
template <bool OUT_BF16>
__global__ __launch_bounds__(kW4Threads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_w4mx_kernel(GemmArgs p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  int tm, tn;
  int split;
  block_of(blockIdx.x, p.tiles_m, p.tiles_n, p.splits, p.group, split, tm, tn);
  const int m0 = tm * 256, n0 = tn * 256;
  const int nk = p.K / 128;
  const int kb_begin = split * p.kb_per_split;
  const int kb_end = min(kb_begin + p.kb_per_split, nk);

  // ---- copy operands (see gen_w4mx_asm.py): buffer resources over the tile's valid rows; the scale
  // arrays hold 4 bytes (one slice's 4 block scales) per row
  const w4_v4i rA = rsrc(p.A + (int64_t)m0 * p.lda, (int64_t)min(256, p.M - m0) * p.lda);
  const w4_v4i rB = rsrc(p.B + (int64_t)n0 * p.ldb, (int64_t)min(256, p.N - n0) * p.ldb);
  const w4_v4i rS = rsrc(p.sA + m0, ((int64_t)nk * p.ldsa - m0) * 4);
  const w4_v4i rX = rsrc(p.sB + n0, ((int64_t)nk * p.N - n0) * 4);
  w4_v8i qa, qb;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    qa[q] = __builtin_amdgcn_readfirstlane((int)(uint32_t)((64 * wave + 8 * q) * p.lda));
    qb[q] = __builtin_amdgcn_readfirstlane((int)(uint32_t)((64 * wave + 8 * q) * p.ldb));
  }
  const int crow = lane >> 3, pch = lane & 7;
  const uint32_t k0 = (uint32_t)kb_begin * 128u;
  uint32_t oa0 = (uint32_t)(crow * p.lda) + (uint32_t)((pch ^ (crow >> 1)) << 4) + k0;
  uint32_t oa1 = (uint32_t)(crow * p.lda) + (uint32_t)((pch ^ (crow >> 1) ^ 4) << 4) + k0;
  uint32_t ob0 = (uint32_t)(crow * p.ldb) + (uint32_t)((pch ^ (crow >> 1)) << 4) + k0;
  uint32_t ob1 = (uint32_t)(crow * p.ldb) + (uint32_t)((pch ^ (crow >> 1) ^ 4) << 4) + k0;
  const uint32_t osa = (uint32_t)lane * 4u;
  uint32_t pfa = (uint32_t)(pf_row(lane, tn, pf_share_a(p)) * p.lda) + k0 + 128u;
  uint32_t pfb = (uint32_t)(pf_row(lane, tm, pf_share_b(p)) * p.ldb) + k0 + 128u;
  int ssp, ssq;                                    // scale offsets of the prefetched slice
  int ssa = __builtin_amdgcn_readfirstlane((int)(((int64_t)kb_begin * p.ldsa + 64 * wave) * 4));
  int ssb = __builtin_amdgcn_readfirstlane((int)(((int64_t)kb_begin * p.N + 64 * wave) * 4));
  const int sstep = __builtin_amdgcn_readfirstlane((int)(p.ldsa * 4));
  const int sstepb = __builtin_amdgcn_readfirstlane((int)(p.N * 4));
  const int mw = wave * 8192, ms = 131072 + 256 * wave;

  // ---- fragment reads (stage 0): lane group g is fed 16-byte chunks g and g + 4 of its row, so that
  // the instruction's 32-element scale block b is the row's MX block b and the lane's own scale byte
  // is that of its row and block g
  const int l16 = lane & 15, g = lane >> 4, sw = l16 >> 1;
  const uint32_t c0 = (uint32_t)((g ^ sw) << 4), c1 = (uint32_t)(((g + 4) ^ sw) << 4);
  const uint32_t aj0 = (uint32_t)((128 * wm + l16) * 128) + c0, aj1 = (uint32_t)((128 * wm + l16) * 128) + c1;
  const uint32_t bj0 = 65536u + (uint32_t)((128 * wn + l16) * 128) + c0;
  const uint32_t bj1 = 65536u + (uint32_t)((128 * wn + l16) * 128) + c1;
  const uint32_t xaj = 131072u + 4u * (uint32_t)(128 * wm + l16) + (uint32_t)g;
  const uint32_t xbj = 131072u + 1024u + 4u * (uint32_t)(128 * wn + l16) + (uint32_t)g;

  // accumulators (zeroed inside the K loop's asm), tile (mi, ni) in a[4 (8 mi + ni) : + 3]; bound as
  // 4-register operands (the compiler moves AGPR values only in pieces of that size)
  w4_v4f acc[64];
  const int n = kb_end - kb_begin;
  int pairs = __builtin_amdgcn_readfirstlane((n - 1) / 2);
  const int rem = __builtin_amdgcn_readfirstlane(n - 2 * ((n - 1) / 2));
  asm volatile(PURO_W4MX_MAINLOOP
               : "=&{a[0:3]}"(acc[0]), "=&{a[4:7]}"(acc[1]), "=&{a[8:11]}"(acc[2]), "=&{a[12:15]}"(acc[3]),
                 "=&{a[16:19]}"(acc[4]), "=&{a[20:23]}"(acc[5]), "=&{a[24:27]}"(acc[6]),
                 "=&{a[28:31]}"(acc[7]), "=&{a[32:35]}"(acc[8]), "=&{a[36:39]}"(acc[9]),
                 "=&{a[40:43]}"(acc[10]), "=&{a[44:47]}"(acc[11]), "=&{a[48:51]}"(acc[12]),
                 "=&{a[52:55]}"(acc[13]), "=&{a[56:59]}"(acc[14]), "=&{a[60:63]}"(acc[15]),
                 "=&{a[64:67]}"(acc[16]), "=&{a[68:71]}"(acc[17]), "=&{a[72:75]}"(acc[18]),
                 "=&{a[76:79]}"(acc[19]), "=&{a[80:83]}"(acc[20]), "=&{a[84:87]}"(acc[21]),
                 "=&{a[88:91]}"(acc[22]), "=&{a[92:95]}"(acc[23]), "=&{a[96:99]}"(acc[24]),
                 "=&{a[100:103]}"(acc[25]), "=&{a[104:107]}"(acc[26]), "=&{a[108:111]}"(acc[27]),
                 "=&{a[112:115]}"(acc[28]), "=&{a[116:119]}"(acc[29]), "=&{a[120:123]}"(acc[30]),
                 "=&{a[124:127]}"(acc[31]), "=&{a[128:131]}"(acc[32]), "=&{a[132:135]}"(acc[33]),
                 "=&{a[136:139]}"(acc[34]), "=&{a[140:143]}"(acc[35]), "=&{a[144:147]}"(acc[36]),
                 "=&{a[148:151]}"(acc[37]), "=&{a[152:155]}"(acc[38]), "=&{a[156:159]}"(acc[39]),
                 "=&{a[160:163]}"(acc[40]), "=&{a[164:167]}"(acc[41]), "=&{a[168:171]}"(acc[42]),
                 "=&{a[172:175]}"(acc[43]), "=&{a[176:179]}"(acc[44]), "=&{a[180:183]}"(acc[45]),
                 "=&{a[184:187]}"(acc[46]), "=&{a[188:191]}"(acc[47]), "=&{a[192:195]}"(acc[48]),
                 "=&{a[196:199]}"(acc[49]), "=&{a[200:203]}"(acc[50]), "=&{a[204:207]}"(acc[51]),
                 "=&{a[208:211]}"(acc[52]), "=&{a[212:215]}"(acc[53]), "=&{a[216:219]}"(acc[54]),
                 "=&{a[220:223]}"(acc[55]), "=&{a[224:227]}"(acc[56]), "=&{a[228:231]}"(acc[57]),
                 "=&{a[232:235]}"(acc[58]), "=&{a[236:239]}"(acc[59]), "=&{a[240:243]}"(acc[60]),
                 "=&{a[244:247]}"(acc[61]), "=&{a[248:251]}"(acc[62]), "=&{a[252:255]}"(acc[63]),
                 "+{v243}"(oa0), "+{v244}"(oa1), "+{v245}"(ob0), "+{v246}"(ob1), "+{v247}"(pfa), "+{v248}"(pfb),
                 [ssa] "+s"(ssa), [ssb] "+s"(ssb), [ssp] "=&s"(ssp), [ssq] "=&s"(ssq), [pairs] "+s"(pairs)
               : [aj0] "v"(aj0), [aj1] "v"(aj1), [bj0] "v"(bj0), [bj1] "v"(bj1), [xaj] "v"(xaj), [xbj] "v"(xbj),
                 [osa] "v"(osa), [rA] "s"(rA), [rB] "s"(rB), [rS] "s"(rS), [rX] "s"(rX), [qa] "{s[64:71]}"(qa),
                 [qb] "{s[72:79]}"(qb), [sstep] "s"(sstep), [sstepb] "s"(sstepb), [mw] "s"(mw), [ms] "s"(ms),
                 [rem] "s"(rem)
               : PURO_W4MX_CLOBBERS, "m0", "scc", "memory");
  (void)ssp;
  (void)ssq;
  w4_epilogue<OUT_BF16, false>(p, smem, wave, lane, m0, n0, split,
                               [&](int mi, int ni, int r) { return acc[8 * mi + ni][r]; });
}

// Every operand offset the kernel forms must fit the 32-bit offsets of a buffer access: A / B rows up
// to 256 x ld bytes past the tile's first row (plus prefetches two slices beyond the last), row-scale
// offsets up to (K / 128 + 2) slices of ldsa floats.
bool w4_supported(const GemmArgs& a) {
  const int64_t lim = int64_t(1) << 32;
  const int64_t nk = a.K / 128;
  return 256 * a.lda + 512 < lim && 256 * a.ldb + 512 < lim && (nk + 2) * a.ldsa * 4 + 1024 < lim;
}

// The MXFP8 kernel's offsets: as the blockwise kernel's, plus the B scales (slices N rows apart).
bool w4mx_supported(const GemmArgs& a) {
  const int64_t lim = int64_t(1) << 32;
  return w4_supported(a) && ((int64_t)a.K / 128 + 2) * a.N * 4 + 1024 < lim;
}

hipError_t launch_w4mx(const GemmArgs& a, bool out_bf16, hipStream_t st) {
  constexpr int kMaxDevices = 64;
  static std::atomic<bool> attr_set[2][kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool known = dev >= 0 && dev < kMaxDevices;
  const void* fn = out_bf16 ? reinterpret_cast<const void*>(&gemm_w4mx_kernel<true>)
                            : reinterpret_cast<const void*>(&gemm_w4mx_kernel<false>);
  if (!known || !attr_set[out_bf16][dev].load(std::memory_order_acquire)) {
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kW4Smem);
    if (e != hipSuccess) return e;
    if (known) attr_set[out_bf16][dev].store(true, std::memory_order_release);
  }
  const dim3 grid((unsigned)(a.tiles_m * a.tiles_n * a.splits));
  if (out_bf16)
    hipLaunchKernelGGL(gemm_w4mx_kernel<true>, grid, dim3(kW4Threads), kW4Smem, st, a);
  else
    hipLaunchKernelGGL(gemm_w4mx_kernel<false>, grid, dim3(kW4Threads), kW4Smem, st, a);
  return hipGetLastError();
}

hipError_t launch_w4(const GemmArgs& a, bool out_bf16, hipStream_t st) {
  // variant: 0 fp32 out, 1 bf16 out, 2 bf16 out with the fused 1x128 quantization (a.q set)
  const int variant = a.q != nullptr ? 2 : (out_bf16 ? 1 : 0);
  if (variant == 2 && !out_bf16) return hipErrorInvalidValue;
  constexpr int kMaxDevices = 64;
  static std::atomic<bool> attr_set[3][kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool known = dev >= 0 && dev < kMaxDevices;
  const void* fn = variant == 2 ? reinterpret_cast<const void*>(&gemm_w4_kernel<true, true>)
                 : variant == 1 ? reinterpret_cast<const void*>(&gemm_w4_kernel<true, false>)
                                : reinterpret_cast<const void*>(&gemm_w4_kernel<false, false>);
  if (!known || !attr_set[variant][dev].load(std::memory_order_acquire)) {
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kW4Smem);
    if (e != hipSuccess) return e;
    if (known) attr_set[variant][dev].store(true, std::memory_order_release);
  }
  const dim3 grid((unsigned)(a.tiles_m * a.tiles_n * a.splits));
  if (variant == 2)
    hipLaunchKernelGGL((gemm_w4_kernel<true, true>), grid, dim3(kW4Threads), kW4Smem, st, a);
  else if (variant == 1)
    hipLaunchKernelGGL((gemm_w4_kernel<true, false>), grid, dim3(kW4Threads), kW4Smem, st, a);
  else
    hipLaunchKernelGGL((gemm_w4_kernel<false, false>), grid, dim3(kW4Threads), kW4Smem, st, a);
  return hipGetLastError();
}

}  // namespace puro

// gfx950 quantizer kernels: 1x128 activation groups, 128x1 token groups written
// transposed (wgrad operands), 128x128 weight blocks (+ optional transposed copy, one
// weight or a batch of them per launch), the dual quantizer (1x128 and transposed 128x1
// codes from one read), its MXFP8 counterpart (32-element blocks, E8M0 scales), and the
// standalone fp32 -> E4M3 cast used to verify the device codec.
//
// All of them are HBM-bound streams (2 B read + 1 B written per element and orientation,
// plus one scale per tile); the kernels use 16-byte coalesced loads and stores, keep the
// tile in registers, reduce amax with DPP / cross-lane moves (and LDS across waves where a
// tile spans waves), and run the per-element work as one fp32 multiply and half a packed
// FP8 convert.
#include "codec.hpp"
#include "internal.hpp"


namespace puro {

// ---------------------------------------------------------------------------------------
// 1x128: one wave covers 4 rows x 1 group per step (16 lanes x 16 B = one 128-element
// group); each wave handles U consecutive groups of its 4 rows, so every lane keeps U
// 16-byte loads in flight.  A workgroup is 4 waves = 16 rows.  Scales of the 4 rows of a
// group are adjacent in the kb-major scale array, so one store instruction writes them.
// ---------------------------------------------------------------------------------------
template <int U>
__global__ __launch_bounds__(256) void quant_1x128_kernel(const uint16_t* __restrict__ x, int64_t M,
                                                          int G, int64_t ldx, uint8_t* __restrict__ q,
                                                          int64_t ldq, float* __restrict__ s,
                                                          int64_t lds, int nkbb) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int ro = lane >> 4;
  const int c = lane & 15;
  const int64_t rb = blockIdx.x / nkbb;
  const int kb0 = (blockIdx.x - (int)(rb * nkbb)) * U;
  const int64_t row = rb * 16 + wave * 4 + ro;
  const bool row_ok = row < M;

  u32x4 v[U];
  const uint16_t* xr = x + row * ldx + c * 8;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int kb = kb0 + u;
    if (row_ok && kb < G)
      v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(xr + (int64_t)kb * 128));
    else
      v[u] = u32x4{0u, 0u, 0u, 0u};
  }
  uint8_t* qr = q + row * ldq + c * 8;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int kb = kb0 + u;
    uint32_t m = pk_max_u16(pk_max_u16(abs2(v[u].x), abs2(v[u].y)), pk_max_u16(abs2(v[u].z), abs2(v[u].w)));
    m = row16_max(hmax16(m));
    float sc, r;
    tile_scale(m, sc, r);
    u32x2 o;
    o.x = cvt4(bf16_lo(v[u].x) * r, bf16_hi(v[u].x) * r, bf16_lo(v[u].y) * r, bf16_hi(v[u].y) * r);
    o.y = cvt4(bf16_lo(v[u].z) * r, bf16_hi(v[u].z) * r, bf16_lo(v[u].w) * r, bf16_hi(v[u].w) * r);
    if (row_ok && kb < G) {
      __builtin_nontemporal_store(o, reinterpret_cast<u32x2*>(qr + (int64_t)kb * 128));
      if (c == 0) s[(int64_t)kb * lds + row] = sc;
    }
  }
}

// Tile order of the transposing quantizers: workgroup b takes token block tb and column
// block g such that runs of `bt` consecutive workgroups cover bt consecutive token blocks of
// one column block.  Each transposed output row then receives bt x 128 contiguous bytes
// from neighbouring workgroups (4 KB with bt = 32) instead of scattered 128-byte pieces,
// which keeps HBM writes within open DRAM pages.  (Measured on MI355X, dual quantizer,
// 16384 x 12288 bf16: 4.6 -> 5.3 TB/s.)
__device__ __forceinline__ void tile_order(int64_t b, int64_t n_col_blocks, int bt, int64_t& tb, int64_t& g) {
  const int64_t run = b / bt, r = b - run * bt;
  tb = (run / n_col_blocks) * bt + r;
  g = run % n_col_blocks;
}

// Token blocks per run: the largest power of two <= 32 dividing the number of token blocks.
static inline int token_run(int64_t nb) {
  int bt = 32;
  while (nb % bt) bt >>= 1;
  return bt;
}

// ---------------------------------------------------------------------------------------
// 128x1, transposed output.  A workgroup owns 128 tokens x 64 columns.  Thread t holds
// 4 consecutive tokens (4*(t>>3) .. +3) x 8 consecutive columns (8*(t&7) .. +7), loaded
// as four coalesced 16-byte reads (8 lanes read one 128-byte row segment).  Column amax:
// packed 16-bit max over the thread's 4 tokens, then across the 8 lanes of the wave
// sharing a column chunk, then across the 4 waves in LDS.  Because a thread holds 4
// consecutive tokens of each of its columns, one packed convert pair yields the 4 output
// bytes of a column directly; the dwords are staged through LDS ([column][token quad],
// odd row stride against bank conflicts) so every output row of 128 bytes is written by
// 8 lanes with 16-byte stores.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void quant_128x1_kernel(const uint16_t* __restrict__ x, int64_t T,
                                                          int64_t C, int64_t ldx,
                                                          uint8_t* __restrict__ qT, int64_t ldqT,
                                                          float* __restrict__ sT, int bt) {
  __shared__ uint32_t red[4][32];
  __shared__ float rsh[64];
  __shared__ uint32_t stage[64 * 33];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int cc = t & 7;
  const int rq = t >> 3;
  int64_t tb, cb;
  tile_order(blockIdx.x, (C + 63) / 64, bt, tb, cb);
  const int64_t c0 = cb * 64;
  const int64_t col = c0 + cc * 8;
  const bool ok = col < C;

  u32x4 v[4];
  const uint16_t* xp = x + (tb * 128 + rq * 4) * ldx + col;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    v[j] = ok ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(xp + j * ldx))
              : u32x4{0u, 0u, 0u, 0u};

  uint32_t m[4];
  m[0] = pk_max_u16(pk_max_u16(abs2(v[0].x), abs2(v[1].x)), pk_max_u16(abs2(v[2].x), abs2(v[3].x)));
  m[1] = pk_max_u16(pk_max_u16(abs2(v[0].y), abs2(v[1].y)), pk_max_u16(abs2(v[2].y), abs2(v[3].y)));
  m[2] = pk_max_u16(pk_max_u16(abs2(v[0].z), abs2(v[1].z)), pk_max_u16(abs2(v[2].z), abs2(v[3].z)));
  m[3] = pk_max_u16(pk_max_u16(abs2(v[0].w), abs2(v[1].w)), pk_max_u16(abs2(v[2].w), abs2(v[3].w)));
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    m[d] = pk_max_u16(m[d], (uint32_t)__shfl_xor((int)m[d], 8));
    m[d] = pk_max_u16(m[d], (uint32_t)__shfl_xor((int)m[d], 16));
    m[d] = pk_max_u16(m[d], (uint32_t)__shfl_xor((int)m[d], 32));
  }
  if (lane < 8) {
#pragma unroll
    for (int d = 0; d < 4; ++d) red[wave][cc * 4 + d] = m[d];
  }
  __syncthreads();
  if (t < 64) {
    const int idx = (t >> 3) * 4 + ((t & 7) >> 1);
    uint32_t w = pk_max_u16(pk_max_u16(red[0][idx], red[1][idx]), pk_max_u16(red[2][idx], red[3][idx]));
    const uint32_t a = (t & 1) ? (w >> 16) : (w & 0xFFFFu);
    float sc, r;
    tile_scale(a, sc, r);
    rsh[t] = r;
    if (c0 + t < C) sT[tb * C + c0 + t] = sc;
  }
  __syncthreads();

#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float r = rsh[cc * 8 + i];
    float e[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w = v[j][i >> 1];
      e[j] = ((i & 1) ? bf16_hi(w) : bf16_lo(w)) * r;
    }
    stage[(cc * 8 + i) * 33 + rq] = cvt4(e[0], e[1], e[2], e[3]);
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int cl = (t >> 3) + 32 * it;
    const int part = t & 7;
    const uint32_t* sp = stage + cl * 33 + part * 4;
    const u32x4 o = {sp[0], sp[1], sp[2], sp[3]};
    if (c0 + cl < C)
      __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(qT + (c0 + cl) * ldqT + tb * 128 + part * 16));
  }
}

// ---------------------------------------------------------------------------------------
// Dual 1x128 + 128x1 quantizer: one read of a bf16 [T, C] tensor yields both the row-wise
// codes (1x128 groups along C; what quant_1x128_kernel writes) and the transposed
// column-wise codes (128x1 groups along T; what quant_128x1_kernel writes), with their
// scales.  A workgroup owns a 128-token x 128-column tile: one 1x128 group per token and
// one 128x1 group per column.  Thread t holds tokens 8*(t>>4) .. +7 x columns 8*(t&15) .. +7
// (eight 16-byte loads; the 16 lanes of a DPP row read one token's 256-byte segment).
//   token amax:  packed max over the thread's 8 columns, then across the 16 lanes of the row;
//   column amax: packed max over the thread's 8 tokens, then across the 4 thread rows of the
//                wave, then across the 4 waves in LDS.
// One thread per token and one per column turn the amaxes into scales (stored) and
// reciprocals (shared through LDS).  Row codes leave directly (16 lanes write a token's
// 128 bytes); transposed codes are staged through LDS ([column][token quad], odd row
// stride) and leave as 128-byte rows written by 8 lanes with 16-byte stores.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void quant_dual_kernel(const uint16_t* __restrict__ x, int64_t T, int64_t C,
                                                         int64_t ldx, uint8_t* __restrict__ q, int64_t ldq,
                                                         float* __restrict__ s, uint8_t* __restrict__ qT,
                                                         int64_t ldqT, float* __restrict__ sT, int bt) {
  __shared__ uint32_t rowmax[64];          // token pairs, packed
  __shared__ uint32_t colred[4][64];       // per wave, column pairs, packed
  __shared__ float rrow[128], rcol[128];
  __shared__ uint32_t stage[128 * 33];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int tc = t & 15, tr = t >> 4;
  int64_t tb, g;
  tile_order(blockIdx.x, C / 128, bt, tb, g);
  const int64_t tok0 = tb * 128 + tr * 8;
  const int64_t col0 = g * 128 + tc * 8;

  u32x4 v[8];
  const uint16_t* xp = x + tok0 * ldx + col0;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(xp + i * ldx));

  // One pass over the thread's values, each |x| pair folded into its token's and its column
  // pair's maxima at once (so no |x| outlives its dword): rm[i] is token i's max over the
  // thread's 8 columns, cm[d] the packed max of columns 8 tc + 2d (low) and 8 tc + 2d + 1 (high)
  // over the thread's 8 tokens.
  uint32_t rm[8], cm[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t a0 = abs2(v[i].x), a1 = abs2(v[i].y), a2 = abs2(v[i].z), a3 = abs2(v[i].w);
    cm[0] = pk_max_u16(cm[0], a0);
    cm[1] = pk_max_u16(cm[1], a1);
    cm[2] = pk_max_u16(cm[2], a2);
    cm[3] = pk_max_u16(cm[3], a3);
    rm[i] = hmax16(pk_max_u16(pk_max_u16(a0, a1), pk_max_u16(a2, a3)));
  }
  // token amax over the tile's 128 columns: rp[k] holds tokens 2k (low half) and 2k+1 (high half)
  uint32_t rp[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) rp[k] = row16_pkmax(rm[2 * k] | (rm[2 * k + 1] << 16));
  if (tc < 4) rowmax[tr * 4 + tc] = tc == 0 ? rp[0] : tc == 1 ? rp[1] : tc == 2 ? rp[2] : rp[3];

  // column amax over the tile's 128 tokens
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t m = cm[d];
    m = pk_max_u16(m, (uint32_t)__shfl_xor((int)m, 16));
    m = pk_max_u16(m, (uint32_t)__shfl_xor((int)m, 32));
    cm[d] = m;
  }
  if (lane < 16) {
#pragma unroll
    for (int d = 0; d < 4; ++d) colred[wave][tc * 4 + d] = cm[d];
  }
  __syncthreads();

  if (t < 128) {                                   // token t of the tile
    const uint32_t w = rowmax[t >> 1];
    float sc, r;
    tile_scale((t & 1) ? (w >> 16) : (w & 0xFFFFu), sc, r);
    rrow[t] = r;
    s[g * T + tb * 128 + t] = sc;
  } else {                                         // column t - 128 of the tile
    const int c = t - 128, idx = c >> 1;
    const uint32_t w = pk_max_u16(pk_max_u16(colred[0][idx], colred[1][idx]),
                                  pk_max_u16(colred[2][idx], colred[3][idx]));
    float sc, r;
    tile_scale((c & 1) ? (w >> 16) : (w & 0xFFFFu), sc, r);
    rcol[c] = r;
    sT[tb * C + g * 128 + c] = sc;
  }
  __syncthreads();

  // row-wise codes: token i's 8 columns -> 8 bytes
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float r = rrow[tr * 8 + i];
    const u32x4 w = v[i];
    u32x2 o;
    o.x = cvt4(bf16_lo(w.x) * r, bf16_hi(w.x) * r, bf16_lo(w.y) * r, bf16_hi(w.y) * r);
    o.y = cvt4(bf16_lo(w.z) * r, bf16_hi(w.z) * r, bf16_lo(w.w) * r, bf16_hi(w.w) * r);
    __builtin_nontemporal_store(o, reinterpret_cast<u32x2*>(q + (tok0 + i) * ldq + col0));
  }
  // column-wise codes: column j's 8 tokens -> two dwords of the staged transposed tile
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float r = rcol[tc * 8 + j];
    float e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t w = v[i][j >> 1];
      e[i] = ((j & 1) ? bf16_hi(w) : bf16_lo(w)) * r;
    }
    stage[(tc * 8 + j) * 33 + 2 * tr] = cvt4(e[0], e[1], e[2], e[3]);
    stage[(tc * 8 + j) * 33 + 2 * tr + 1] = cvt4(e[4], e[5], e[6], e[7]);
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int cl = (t >> 3) + 32 * it;
    const int part = t & 7;
    const uint32_t* sp = stage + cl * 33 + part * 4;
    const u32x4 o = {sp[0], sp[1], sp[2], sp[3]};
    __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(qT + (g * 128 + cl) * ldqT + tb * 128 + part * 16));
  }
}

// ---------------------------------------------------------------------------------------
// MXFP8 dual quantizer (OCP Microscaling format with E4M3 elements; the pages' Blackwell
// path): blocks of 32 elements along the contraction axis share one E8M0 scale
// X = 2^(floor(log2 amax) - 8) (8: exponent of E4M3's largest normal, 448 = 1.75 * 2^8),
// clamped to [2^-127, 2^127]; each element becomes E4M3_rne_sat(x / X).  Like the blockwise
// dual kernel, one read of x [T, C] yields the row-wise codes (blocks along C, for FWD /
// DGRAD) and the transposed column-wise codes (blocks along T, for WGRAD).  Scales are
// written as bytes [C/128][T][4] and [T/128][C][4]: the four block scales of one 128-deep
// slice of a row are adjacent.
// Tile and thread layout as quant_dual_kernel (128 x 128, thread = 8 tokens x 8 columns):
//   a row block (32 columns of one token) is one DPP quad of lanes: quad max;
//   a column block (32 tokens of one column) is one wave's 4 thread rows: xor 16, 32.
// The scale code is read off the amax's bf16 exponent field E: max(E - 8, 0), or 255 (NaN
// scale) for a NaN or infinity.  x / X is the exact multiply by 2^(127 - code), built from
// its exponent field; |x / X| < 512, clamped to +-448 before the convert (saturation).
// Blocks with the NaN scale get NaN codes throughout.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t mx_code(uint32_t amax_bits) {
  const uint32_t e = amax_bits >> 7;           // sign already cleared
  return e == 255u ? 255u : (e > 8u ? e - 8u : 0u);
}
__device__ __forceinline__ float mx_mul(uint32_t code) {
  return code == 255u ? __builtin_nanf("") : __uint_as_float((254u - code) << 23);
}
__device__ __forceinline__ float clamp448(float v) { return __builtin_amdgcn_fmed3f(v, -kE4M3Max, kE4M3Max); }

__global__ __launch_bounds__(256) void mx_quant_dual_kernel(const uint16_t* __restrict__ x, int64_t T, int64_t C,
                                                            int64_t ldx, uint8_t* __restrict__ q, int64_t ldq,
                                                            uint8_t* __restrict__ xs, uint8_t* __restrict__ qT,
                                                            int64_t ldqT, uint8_t* __restrict__ xsT, int bt) {
  __shared__ uint8_t rowsc[128 * 4];       // [token][block]
  __shared__ uint8_t colsc[128 * 4];       // [column][block]
  __shared__ uint32_t stage[128 * 33];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int tc = t & 15, tr = t >> 4;
  int64_t tb, g;
  tile_order(blockIdx.x, C / 128, bt, tb, g);
  const int64_t tok0 = tb * 128 + tr * 8;
  const int64_t col0 = g * 128 + tc * 8;

  u32x4 v[8];
  const uint16_t* xp = x + tok0 * ldx + col0;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(xp + i * ldx));

  // row blocks: amax of tokens 2k (low half) / 2k+1 (high half) over the quad's 32 columns
  uint32_t rcode[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t m2[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const u32x4 w = v[2 * k + e];
      m2[e] = hmax16(pk_max_u16(pk_max_u16(abs2(w.x), abs2(w.y)), pk_max_u16(abs2(w.z), abs2(w.w))));
    }
    uint32_t p = m2[0] | (m2[1] << 16);
    p = pk_max_u16(p, dpp<kDppQuadXor1>(p));
    p = pk_max_u16(p, dpp<kDppQuadXor2>(p));
    rcode[2 * k] = mx_code(p & 0xFFFFu);
    rcode[2 * k + 1] = mx_code(p >> 16);
  }
  // column blocks: amax of columns 8 tc + 2d (low) / + 1 (high) over the wave's 32 tokens
  uint32_t ccode[8];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t m = abs2(v[0][d]);
#pragma unroll
    for (int i = 1; i < 8; ++i) m = pk_max_u16(m, abs2(v[i][d]));
    m = pk_max_u16(m, (uint32_t)__shfl_xor((int)m, 16));
    m = pk_max_u16(m, (uint32_t)__shfl_xor((int)m, 32));
    ccode[2 * d] = mx_code(m & 0xFFFFu);
    ccode[2 * d + 1] = mx_code(m >> 16);
  }
  if ((tc & 3) == 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) rowsc[(tr * 8 + i) * 4 + (tc >> 2)] = (uint8_t)rcode[i];
  }
  if (lane < 16) {
#pragma unroll
    for (int j = 0; j < 8; ++j) colsc[(tc * 8 + j) * 4 + wave] = (uint8_t)ccode[j];
  }

  // row-wise codes: token i's 8 columns -> 8 bytes
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float r = mx_mul(rcode[i]);
    const u32x4 w = v[i];
    u32x2 o;
    o.x = cvt4(clamp448(bf16_lo(w.x) * r), clamp448(bf16_hi(w.x) * r), clamp448(bf16_lo(w.y) * r),
               clamp448(bf16_hi(w.y) * r));
    o.y = cvt4(clamp448(bf16_lo(w.z) * r), clamp448(bf16_hi(w.z) * r), clamp448(bf16_lo(w.w) * r),
               clamp448(bf16_hi(w.w) * r));
    if (rcode[i] == 255u) o |= 0x7F7F7F7Fu;
    __builtin_nontemporal_store(o, reinterpret_cast<u32x2*>(q + (tok0 + i) * ldq + col0));
  }
  // column-wise codes: column j's 8 tokens -> two dwords of the staged transposed tile
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float r = mx_mul(ccode[j]);
    float e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t w = v[i][j >> 1];
      e[i] = clamp448(((j & 1) ? bf16_hi(w) : bf16_lo(w)) * r);
    }
    uint32_t lo = cvt4(e[0], e[1], e[2], e[3]), hi = cvt4(e[4], e[5], e[6], e[7]);
    if (ccode[j] == 255u) {
      lo |= 0x7F7F7F7Fu;
      hi |= 0x7F7F7F7Fu;
    }
    stage[(tc * 8 + j) * 33 + 2 * tr] = lo;
    stage[(tc * 8 + j) * 33 + 2 * tr + 1] = hi;
  }
  __syncthreads();
  if (t < 128)
    reinterpret_cast<uint32_t*>(xs)[g * T + tb * 128 + t] = reinterpret_cast<const uint32_t*>(rowsc)[t];
  else
    reinterpret_cast<uint32_t*>(xsT)[tb * C + g * 128 + (t - 128)] = reinterpret_cast<const uint32_t*>(colsc)[t - 128];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int cl = (t >> 3) + 32 * it;
    const int part = t & 7;
    const uint32_t* sp = stage + cl * 33 + part * 4;
    const u32x4 o = {sp[0], sp[1], sp[2], sp[3]};
    __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(qT + (g * 128 + cl) * ldqT + tb * 128 + part * 16));
  }
}

// ---------------------------------------------------------------------------------------
// 128x128 weight blocks.  One workgroup per block; thread t holds rows 8*(t>>4) .. +7 of
// the block at columns 8*(t&15) .. +7 (8 coalesced 16-byte loads).  Block amax: packed
// max in registers, DPP/cross-lane max in the wave, LDS across the 4 waves.  The thread's
// 8x8 sub-block is converted row-wise for q (16 lanes write a row's 128 bytes) and
// column-wise for the transposed copy qT, staged through LDS like the transposing activation
// quantizers so that qT rows leave as 128-byte segments.  Workgroups take the blocks in runs
// of consecutive N blocks of one K block (tile_order), so each qT row is written in long
// contiguous runs.
// ---------------------------------------------------------------------------------------
// One 128 x 128 block (number blk of the weight's tile order) of one weight.
__device__ __forceinline__ void quant_128x128_block(const uint16_t* __restrict__ w, int64_t N, int64_t K, int64_t ldw,
                                                    uint8_t* __restrict__ q, int64_t ldq, float* __restrict__ s,
                                                    uint8_t* __restrict__ qT, int64_t ldqT, float* __restrict__ sT,
                                                    int bt, int64_t blk) {
  __shared__ uint32_t red[4];
  __shared__ uint32_t stage[128 * 33];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int cc = t & 15;
  const int rg = t >> 4;
  int64_t nb, kb;
  tile_order(blk, K >> 7, bt, nb, kb);
  const int64_t n0 = nb * 128 + rg * 8;
  const int64_t k0 = kb * 128 + cc * 8;

  u32x4 v[8];
  const uint16_t* wp = w + n0 * ldw + k0;
#pragma unroll
  for (int p = 0; p < 8; ++p)
    v[p] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wp + p * ldw));

  uint32_t m = 0;
#pragma unroll
  for (int p = 0; p < 8; ++p)
    m = pk_max_u16(m, pk_max_u16(pk_max_u16(abs2(v[p].x), abs2(v[p].y)), pk_max_u16(abs2(v[p].z), abs2(v[p].w))));
  m = wave_max(hmax16(m));
  if (lane == 0) red[wave] = m;
  __syncthreads();
  m = umax(umax(red[0], red[1]), umax(red[2], red[3]));
  float sc, r;
  tile_scale(m, sc, r);
  if (t == 0) {
    const int64_t KB = K >> 7, NB = N >> 7;
    s[nb * KB + kb] = sc;
    if (sT) sT[kb * NB + nb] = sc;
  }

  // row p's codes: rc[p][0] = columns 0-3, rc[p][1] = columns 4-7 of the thread's 8 (byte c = column c)
  uint8_t* qp = q + n0 * ldq + k0;
  uint32_t rc[8][2];
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const u32x4 x = v[p];
    rc[p][0] = cvt4(bf16_lo(x.x) * r, bf16_hi(x.x) * r, bf16_lo(x.y) * r, bf16_hi(x.y) * r);
    rc[p][1] = cvt4(bf16_lo(x.z) * r, bf16_hi(x.z) * r, bf16_lo(x.w) * r, bf16_hi(x.w) * r);
    const u32x2 o = {rc[p][0], rc[p][1]};
    __builtin_nontemporal_store(o, reinterpret_cast<u32x2*>(qp + p * ldq));
  }
  if (qT) {   // (uniform branch: qT is a kernel argument)
    // The block has one scale, so the transposed codes are the same bytes: each 4 x 4 byte square
    // (rows 4u .. 4u+3, columns 4h .. 4h+3) is transposed with byte permutes (v_perm_b32 picks
    // bytes 0-3 from its second operand and 4-7 from its first), giving column 4h + c's codes of
    // rows 4u .. 4u+3 as one dword of the staged [column][row quad] tile.
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t d0 = rc[4 * u][h], d1 = rc[4 * u + 1][h], d2 = rc[4 * u + 2][h], d3 = rc[4 * u + 3][h];
        const uint32_t p01lo = __builtin_amdgcn_perm(d1, d0, 0x05010400u);   // d0.b0 d1.b0 d0.b1 d1.b1
        const uint32_t p01hi = __builtin_amdgcn_perm(d1, d0, 0x07030602u);   // d0.b2 d1.b2 d0.b3 d1.b3
        const uint32_t p23lo = __builtin_amdgcn_perm(d3, d2, 0x05010400u);
        const uint32_t p23hi = __builtin_amdgcn_perm(d3, d2, 0x07030602u);
        uint32_t* col = stage + (cc * 8 + 4 * h) * 33 + 2 * rg + u;
        col[0] = __builtin_amdgcn_perm(p23lo, p01lo, 0x05040100u);           // byte 0 of d0 .. d3
        col[33] = __builtin_amdgcn_perm(p23lo, p01lo, 0x07060302u);          // byte 1
        col[66] = __builtin_amdgcn_perm(p23hi, p01hi, 0x05040100u);          // byte 2
        col[99] = __builtin_amdgcn_perm(p23hi, p01hi, 0x07060302u);          // byte 3
      }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int cl = (t >> 3) + 32 * it;
      const int part = t & 7;
      const uint32_t* sp = stage + cl * 33 + part * 4;
      const u32x4 o = {sp[0], sp[1], sp[2], sp[3]};
      __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(qT + (kb * 128 + cl) * ldqT + nb * 128 + part * 16));
    }
  }
}

__global__ __launch_bounds__(256) void quant_128x128_kernel(const uint16_t* __restrict__ w, int64_t N,
                                                            int64_t K, int64_t ldw,
                                                            uint8_t* __restrict__ q, int64_t ldq,
                                                            float* __restrict__ s,
                                                            uint8_t* __restrict__ qT, int64_t ldqT,
                                                            float* __restrict__ sT, int bt) {
  quant_128x128_block(w, N, K, ldw, q, ldq, s, qT, ldqT, sT, bt, blockIdx.x);
}

// Several weights in one launch: job j owns blocks first[j] .. first[j + 1) - 1 (a wave-uniform
// scan over at most kMaxWeightJobs jobs), each in its own tile order.
__global__ __launch_bounds__(256) void quant_128x128_batch_kernel(WeightJobs jobs) {
  int j = jobs.n - 1;
  while (j > 0 && (int64_t)blockIdx.x < jobs.job[j].first) --j;
  const WeightJob& b = jobs.job[j];
  quant_128x128_block(b.w, b.N, b.K, b.ldw, b.q, b.ldq, b.s, b.qT, b.ldqT, b.sT, b.bt,
                      (int64_t)blockIdx.x - b.first);
}

// ---------------------------------------------------------------------------------------
// Standalone saturating cast: 4 floats -> one dword of codes per step.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void cast_e4m3_kernel(const float* __restrict__ v, int64_t n,
                                                        uint8_t* __restrict__ q) {
  const int64_t n4 = n >> 2;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    const float4 f = reinterpret_cast<const float4*>(v)[i];
    reinterpret_cast<uint32_t*>(q)[i] = cvt4(sat448(f.x), sat448(f.y), sat448(f.z), sat448(f.w));
  }
  const int64_t tail = n & 3;
  if (tail && blockIdx.x == 0 && threadIdx.x < tail) {
    const int64_t i = n4 * 4 + threadIdx.x;
    q[i] = (uint8_t)(cvt2_lo(sat448(v[i]), 0.0f, 0u) & 0xFFu);
  }
}

// ---------------------------------------------------------------------------------------
// Host-side launchers (shapes already validated by the ABI layer).
// ---------------------------------------------------------------------------------------
hipError_t launch_quant_1x128(const void* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q,
                              int64_t ldq, float* s, hipStream_t st, int64_t lds) {
  constexpr int U = 4;
  const int G = (int)(K / 128);
  const int nkbb = (G + U - 1) / U;
  const int64_t nrb = (M + 15) / 16;
  const int64_t blocks = nrb * nkbb;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(quant_1x128_kernel<U>, dim3((unsigned)blocks), dim3(256), 0, st,
                     static_cast<const uint16_t*>(x), M, G, ldx, q, ldq, s, lds > 0 ? lds : M, nkbb);
  return hipGetLastError();
}

hipError_t launch_quant_128x1(const void* x, int64_t T, int64_t C, int64_t ldx, uint8_t* qT,
                              int64_t ldqT, float* sT, hipStream_t st) {
  const int64_t nc = (C + 63) / 64, nb = T / 128;
  if (nc * nb > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(quant_128x1_kernel, dim3((unsigned)(nc * nb)), dim3(256), 0, st,
                     static_cast<const uint16_t*>(x), T, C, ldx, qT, ldqT, sT, token_run(nb));
  return hipGetLastError();
}

hipError_t launch_quant_dual(const void* x, int64_t T, int64_t C, int64_t ldx, uint8_t* q, int64_t ldq,
                             float* s, uint8_t* qT, int64_t ldqT, float* sT, hipStream_t st) {
  const int64_t nb = T / 128, ng = C / 128;
  if (nb * ng > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(quant_dual_kernel, dim3((unsigned)(nb * ng)), dim3(256), 0, st,
                     static_cast<const uint16_t*>(x), T, C, ldx, q, ldq, s, qT, ldqT, sT, token_run(nb));
  return hipGetLastError();
}

hipError_t launch_mx_quant_dual(const void* x, int64_t T, int64_t C, int64_t ldx, uint8_t* q, int64_t ldq,
                                uint8_t* xs, uint8_t* qT, int64_t ldqT, uint8_t* xsT, hipStream_t st) {
  const int64_t nb = T / 128, ng = C / 128;
  if (nb * ng > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(mx_quant_dual_kernel, dim3((unsigned)(nb * ng)), dim3(256), 0, st,
                     static_cast<const uint16_t*>(x), T, C, ldx, q, ldq, xs, qT, ldqT, xsT, token_run(nb));
  return hipGetLastError();
}

hipError_t launch_quant_128x128_batch(const WeightJob* jobs, int n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  if (n > kMaxWeightJobs) return hipErrorInvalidValue;
  WeightJobs a;
  int64_t total = 0;
  a.n = 0;
  for (int i = 0; i < n; ++i) {
    const int64_t blocks = (jobs[i].N / 128) * (jobs[i].K / 128);
    if (blocks == 0) continue;                   // empty weights take no blocks
    a.job[a.n] = jobs[i];
    a.job[a.n].bt = token_run(jobs[i].N / 128);
    a.job[a.n].first = total;
    total += blocks;
    ++a.n;
  }
  if (a.n == 0) return hipSuccess;
  if (total > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(quant_128x128_batch_kernel, dim3((unsigned)total), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_quant_128x128(const void* w, int64_t N, int64_t K, int64_t ldw, uint8_t* q,
                                int64_t ldq, float* s, uint8_t* qT, int64_t ldqT, float* sT,
                                hipStream_t st) {
  const int64_t nb = N / 128, kb = K / 128;
  if (nb * kb > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(quant_128x128_kernel, dim3((unsigned)(nb * kb)), dim3(256), 0, st,
                     static_cast<const uint16_t*>(w), N, K, ldw, q, ldq, s, qT, ldqT, sT, token_run(nb));
  return hipGetLastError();
}

hipError_t launch_cast_e4m3(const float* v, int64_t n, uint8_t* q, hipStream_t st) {
  int64_t blocks = ((n >> 2) + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(cast_e4m3_kernel, dim3((unsigned)blocks), dim3(256), 0, st, v, n, q);
  return hipGetLastError();
}

}  // namespace puro

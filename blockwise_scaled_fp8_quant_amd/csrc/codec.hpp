// Device-side E4M3 codec and tile-scale helpers shared by the gfx950 quantizer kernels and
// the GEMM epilogue's fused 1x128 output quantization.
//
// Tile numerics (the pages fix only "FP8, activations per 128, weights per 128x128
// block, one scale per block"; the readings below are this library's):
//   amax      = max |x| over the tile, taken on the bf16 bit patterns with the sign
//               cleared (for non-NaN values the unsigned integer order of those bits is
//               the order of the magnitudes, so the max is exact; a NaN sorts above
//               +inf and propagates).
//   amax_eff  = max(amax, 2^-96)   (bf16 0x0F80; keeps s normal and r finite)
//   s         = fl32(amax_eff / 448)       stored scale
//   r         = fl32(448 / amax_eff)       per-element multiplier
//   code      = E4M3_rne_sat(fl32(x * r))
// The divisions are IEEE correctly rounded: hipcc's default fp32 division on gfx950
// (no fast-math, no approximate reciprocal) is the correctly rounded sequence.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace puro {

constexpr float kE4M3Max = 448.0f;
constexpr uint32_t kAmaxFloorBf16 = 0x0F80u;   // 2^-96 as bf16 bits

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 16-bit lanes of a dword: unsigned max per half (v_pk_max_u16).
typedef unsigned short us2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  us2 va = __builtin_bit_cast(us2, a);
  us2 vb = __builtin_bit_cast(us2, b);
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(va, vb));
}

// |x| bits of two packed bf16 values.
__device__ __forceinline__ uint32_t abs2(uint32_t w) { return w & 0x7FFF7FFFu; }

// max of the two 16-bit halves, as a 32-bit value.
__device__ __forceinline__ uint32_t hmax16(uint32_t w) {
  uint32_t lo = w & 0xFFFFu, hi = w >> 16;
  return lo > hi ? lo : hi;
}

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// Scale and reciprocal from the amax bf16 bits (sign already cleared).
__device__ __forceinline__ void tile_scale(uint32_t amax_bits, float& s, float& r) {
  const uint32_t eff = umax(amax_bits, kAmaxFloorBf16);
  const float a = __uint_as_float(eff << 16);
  s = a / kE4M3Max;
  r = kE4M3Max / a;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two fp32 -> E4M3 codes into the low (hi_word = false) or high half of `old`.
// v_cvt_pk_fp8_f32 rounds to nearest even (OCP E4M3 on gfx950).  The quantizers only
// feed it |v| <= 448 * (1 + 2^-23), which rounds to at most 448, so the saturation
// question never arises there; the explicit clamp below makes the standalone cast
// saturating for every finite or infinite input as well (NaN passes through).
__device__ __forceinline__ float sat448(float v) {
  // fminf/fmaxf would turn NaN into +-448; compare on the magnitude instead.
  const float a = __builtin_fabsf(v);
  return a > kE4M3Max ? __builtin_copysignf(kE4M3Max, v) : v;
}

__device__ __forceinline__ uint32_t cvt2_lo(float a, float b, uint32_t old) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, false);
}
__device__ __forceinline__ uint32_t cvt2_hi(float a, float b, uint32_t old) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, true);
}

// Four scaled values -> one dword of codes (byte i = element i).
__device__ __forceinline__ uint32_t cvt4(float a, float b, float c, float d) {
  uint32_t w = cvt2_lo(a, b, 0u);
  return cvt2_hi(c, d, w);
}

// DPP helpers (row = 16 lanes).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  // every row and bank enabled and every control used here a permutation within a row: each lane
  // receives a value, so no "old" operand (and no register zeroed for it) is needed
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}
constexpr int kDppQuadXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;  // lane i <-> 7-i within each 8 lanes
constexpr int kDppRowMirror = 0x140;      // lane i <-> 15-i within each 16 lanes

// Max over the 16 lanes of a DPP row (every lane of the row receives the result).
__device__ __forceinline__ uint32_t row16_max(uint32_t v) {
  v = umax(v, dpp<kDppQuadXor1>(v));
  v = umax(v, dpp<kDppQuadXor2>(v));
  v = umax(v, dpp<kDppRowHalfMirror>(v));
  v = umax(v, dpp<kDppRowMirror>(v));
  return v;
}

// Packed 16-bit max over the 16 lanes of a DPP row (every lane receives the result).
__device__ __forceinline__ uint32_t row16_pkmax(uint32_t v) {
  v = pk_max_u16(v, dpp<kDppQuadXor1>(v));
  v = pk_max_u16(v, dpp<kDppQuadXor2>(v));
  v = pk_max_u16(v, dpp<kDppRowHalfMirror>(v));
  v = pk_max_u16(v, dpp<kDppRowMirror>(v));
  return v;
}

// Max over all 64 lanes of the wave.
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  v = row16_max(v);
  v = umax(v, (uint32_t)__shfl_xor((int)v, 16));
  v = umax(v, (uint32_t)__shfl_xor((int)v, 32));
  return v;
}

}  // namespace puro

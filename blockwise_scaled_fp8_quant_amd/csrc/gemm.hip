// gfx950 blockwise-scaled FP8 GEMM with per-128-slice fp32 promotion.
//
//   C[i,j] = sum_kb  sA(i,kb) * sB(j,kb) * P_kb[i,j],   P_kb[i,j] = sum_{k in slice kb} A[i,k] B[j,k]
//
// P_kb is produced by the FP8 matrix cores (v_mfma_f32_32x32x64_f8f6f4, E4M3 x E4M3 ->
// fp32; two instructions cover one 128-deep slice of a 32x32 output tile), and the
// promotion C_acc += P_kb * (sA * sB) runs on the vector ALUs into a separate fp32
// accumulator, as the DeepSeek-V3-style fine-grained scheme the pages follow prescribes
// (ModelScope write-up on Puro-2B, section 精度).
//
// Operand roles inside the MFMA are swapped (the B tile is the instruction's A operand)
// so that every lane owns ONE output row i and 16 output columns: the activation scale
// sA(i,kb) is then one register per lane and slice, and for the 128x128-block weight
// scales of FWD/DGRAD the whole scale product is a single multiply per lane and slice.
#include <hip/hip_runtime.h>

#include "internal.hpp"

namespace puro {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef uint32_t g_u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t g_u32x2 __attribute__((ext_vector_type(2)));
typedef float g_f32x4 __attribute__((ext_vector_type(4)));

// D = X * Y + Cin for X: 32x64 (lanes index rows), Y: 64x32 (lanes index columns), E4M3.
// Zero scale operands select the unscaled instruction.
__device__ __forceinline__ v16f mfma_32x32x64_e4m3(v8i x, v8i y, v16f c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x, y, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;   // quiet NaN
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ v8i join(g_u32x4 a, g_u32x4 b) {
  v8i r;
  r[0] = (int)a[0]; r[1] = (int)a[1]; r[2] = (int)a[2]; r[3] = (int)a[3];
  r[4] = (int)b[0]; r[5] = (int)b[1]; r[6] = (int)b[2]; r[7] = (int)b[3];
  return r;
}

// 16-byte chunk swizzle of a [rows][128 B] LDS tile: chunk c of row r lives at c ^ (r & 7),
// so 8 consecutive rows reading the same logical chunk hit 8 different bank groups.
__device__ __forceinline__ int swz(int r, int c) { return c ^ (r & 7); }

// ---------------------------------------------------------------------------------------
// v0: 128x128 block tile, 4 waves in a 2x2 grid of 64x64 wave tiles (2x2 MFMA tiles of
// 32x32 each), one 128-deep slice per step; the next slice is prefetched into registers
// while the current one is multiplied.
// ---------------------------------------------------------------------------------------
template <int MODE, bool OUT_BF16>
__global__ __launch_bounds__(256) void gemm_v0_kernel(int M, int N, int K, const uint8_t* __restrict__ A,
                                                      int64_t lda, const float* __restrict__ sA,
                                                      const uint8_t* __restrict__ B, int64_t ldb,
                                                      const float* __restrict__ sB, void* __restrict__ Cv,
                                                      int64_t ldc) {
  __shared__ __attribute__((aligned(16))) uint8_t As[128 * 128];
  __shared__ __attribute__((aligned(16))) uint8_t Bs[128 * 128];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * 128, n0 = blockIdx.x * 128;
  const int nk = K >> 7;
  const int gc = t & 7, gr = t >> 3;
  const uint8_t* Ag = A + (int64_t)(m0 + gr) * lda + gc * 16;
  const uint8_t* Bg = B + (int64_t)(n0 + gr) * ldb + gc * 16;
  const int l32 = lane & 31, h = lane >> 5;

  g_u32x4 ra[4], rb[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    ra[p] = *reinterpret_cast<const g_u32x4*>(Ag + (int64_t)p * 32 * lda);
    rb[p] = *reinterpret_cast<const g_u32x4*>(Bg + (int64_t)p * 32 * ldb);
  }

  v16f acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.0f;
  const v16f zero = acc[0][0];

  for (int kb = 0; kb < nk; ++kb) {
    __syncthreads();
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int r = gr + 32 * p;
      *reinterpret_cast<g_u32x4*>(As + r * 128 + swz(r, gc) * 16) = ra[p];
      *reinterpret_cast<g_u32x4*>(Bs + r * 128 + swz(r, gc) * 16) = rb[p];
    }
    __syncthreads();
    if (kb + 1 < nk) {
      const int64_t ko = (int64_t)(kb + 1) * 128;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        ra[p] = *reinterpret_cast<const g_u32x4*>(Ag + (int64_t)p * 32 * lda + ko);
        rb[p] = *reinterpret_cast<const g_u32x4*>(Bg + (int64_t)p * 32 * ldb + ko);
      }
    }

    float sa[2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) sa[mi] = sA[(int64_t)kb * M + m0 + wm * 64 + mi * 32 + l32];
    float sbb = 0.0f;
    g_f32x4 sbw[2][4];
    if (MODE != 2) {
      sbb = sB[(int64_t)(n0 >> 7) * (K >> 7) + kb];
    } else {
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          sbw[ni][g] = *reinterpret_cast<const g_f32x4*>(sB + (int64_t)kb * N + n0 + wn * 64 + ni * 32 + 8 * g + 4 * h);
    }

    v8i af[2][2], bf[2][2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
      const int r = wm * 64 + mi * 32 + l32;
      g_u32x4 c[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) c[j] = *reinterpret_cast<const g_u32x4*>(As + r * 128 + swz(r, 4 * h + j) * 16);
      af[mi][0] = join(c[0], c[1]);
      af[mi][1] = join(c[2], c[3]);
    }
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      const int r = wn * 64 + ni * 32 + l32;
      g_u32x4 c[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) c[j] = *reinterpret_cast<const g_u32x4*>(Bs + r * 128 + swz(r, 4 * h + j) * 16);
      bf[ni][0] = join(c[0], c[1]);
      bf[ni][1] = join(c[2], c[3]);
    }

#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        v16f p = mfma_32x32x64_e4m3(bf[ni][0], af[mi][0], zero);
        p = mfma_32x32x64_e4m3(bf[ni][1], af[mi][1], p);
        if (MODE != 2) {
          const float sc = sa[mi] * sbb;
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[mi][ni][v] = __builtin_fmaf(p[v], sc, acc[mi][ni][v]);
        } else {
#pragma unroll
          for (int v = 0; v < 16; ++v)
            acc[mi][ni][v] = __builtin_fmaf(p[v], sa[mi] * sbw[ni][v >> 2][v & 3], acc[mi][ni][v]);
        }
      }
    }
  }

  // Epilogue: lane owns row i, columns j0 + 8g + {0..3}.
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
    const int64_t i = m0 + wm * 64 + mi * 32 + l32;
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      const int64_t j0 = n0 + wn * 64 + ni * 32 + 4 * h;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t j = j0 + 8 * g;
        if (OUT_BF16) {
          g_u32x2 o;
          o[0] = bf16_rne(acc[mi][ni][4 * g + 0]) | (bf16_rne(acc[mi][ni][4 * g + 1]) << 16);
          o[1] = bf16_rne(acc[mi][ni][4 * g + 2]) | (bf16_rne(acc[mi][ni][4 * g + 3]) << 16);
          *reinterpret_cast<g_u32x2*>(static_cast<uint16_t*>(Cv) + i * ldc + j) = o;
        } else {
          g_f32x4 o = {acc[mi][ni][4 * g + 0], acc[mi][ni][4 * g + 1], acc[mi][ni][4 * g + 2],
                       acc[mi][ni][4 * g + 3]};
          *reinterpret_cast<g_f32x4*>(static_cast<float*>(Cv) + i * ldc + j) = o;
        }
      }
    }
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

size_t gemm_workspace_bytes(int, int64_t, int64_t, int64_t) { return 0; }

template <int MODE>
static hipError_t launch_mode(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                              const float* sA, const uint8_t* B, int64_t ldb, const float* sB,
                              void* C, int64_t ldc, bool out_bf16, hipStream_t st) {
  const dim3 grid((unsigned)(N / 128), (unsigned)(M / 128));
  if (out_bf16)
    hipLaunchKernelGGL((gemm_v0_kernel<MODE, true>), grid, dim3(256), 0, st, (int)M, (int)N, (int)K, A,
                       lda, sA, B, ldb, sB, C, ldc);
  else
    hipLaunchKernelGGL((gemm_v0_kernel<MODE, false>), grid, dim3(256), 0, st, (int)M, (int)N, (int)K, A,
                       lda, sA, B, ldb, sB, C, ldc);
  return hipGetLastError();
}

hipError_t launch_gemm(int mode, int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                       const float* sA, const uint8_t* B, int64_t ldb, const float* sB, void* C,
                       int64_t ldc, bool out_bf16, void*, size_t, hipStream_t st) {
  if (K == 0) {
    const int64_t es = out_bf16 ? 2 : 4;
    const int64_t gy = M < 65535 ? M : 65535;
    hipLaunchKernelGGL(zero_fill_kernel, dim3(8, (unsigned)gy), dim3(256), 0, st, C, M, N * es, ldc * es);
    return hipGetLastError();
  }
  if (N / 128 > 0x7FFFFFFF || M / 128 > 65535) return hipErrorInvalidConfiguration;
  switch (mode) {
    case 0: return launch_mode<0>(M, N, K, A, lda, sA, B, ldb, sB, C, ldc, out_bf16, st);
    case 1: return launch_mode<1>(M, N, K, A, lda, sA, B, ldb, sB, C, ldc, out_bf16, st);
    default: return launch_mode<2>(M, N, K, A, lda, sA, B, ldb, sB, C, ldc, out_bf16, st);
  }
}

}  // namespace puro

"""MXFP8 microscaling quantization and GEMM, written out on the CPU (the pages' Blackwell path).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this module.

What the pages fix: the agihunt digest ("清华用消费级 5090 花 6890 美元从零训 2B…", section
方法, FP8 bullet) says that on Blackwell the linear layers run MXFP8 instead of the 1x128 /
128x128 scheme.  They give no further detail, so this module follows the public OCP
Microscaling (MX) v1.0 format with FP8 E4M3 elements:

  * a block is 32 consecutive elements along the contraction axis of the consuming GEMM
    (the reading R8 of the blockwise scheme carried over);
  * each block has one shared scale X = 2^E stored as an E8M0 byte (code = E + 127; code
    255 is NaN; there is no zero and no sign);
  * E = floor(log2(amax)) - 8, where 8 is the exponent of E4M3's largest normal value
    (448 = 1.75 * 2^8), so the block's largest element lands in [256, 512) after scaling;
    E is clamped into the E8M0 range [-127, 127];
  * each element becomes code = E4M3_rne_sat(x / X): round to nearest even, saturating to
    +-448 (values in [448, 512) X saturate);
  * readings where the spec leaves room: an all-zero block gets E = -127 (code 0); a block
    holding a NaN or an infinity gets the NaN scale (code 255).  Non-finite input is outside
    the bit-exact contract.

Layouts (the library's): codes [R, K] row-major like the blockwise scheme; scales uint8
[K/128][R][4]: byte (kb, r, j) is the scale of row r, elements 128 kb + 32 j .. + 31 (the
four blocks of one 128-deep slice of a row are adjacent).

Steps in the order the method takes them: per block amax -> shared exponent -> scaled cast
of every element -> emit codes and scales.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

from . import e4m3
from .quant import bf16_bits_to_f32

BLOCK = 32
EMAX_E4M3 = 8          # 448 = 1.75 * 2^8
E8M0_BIAS = 127
E8M0_NAN = 255


def e8m0_decode(codes: np.ndarray) -> np.ndarray:
    """float64 value of E8M0 bytes: 2^(code - 127); code 255 is NaN."""
    c = np.asarray(codes, dtype=np.int64)
    v = np.ldexp(1.0, c - E8M0_BIAS)
    return np.where(c == E8M0_NAN, np.nan, v)


def shared_exponent_code(amax: np.ndarray) -> np.ndarray:
    """E8M0 code of floor(log2(amax)) - 8, clamped to [-127, 127]; 0 for amax == 0, 255 for
    NaN or infinity.  floor(log2 a) comes from frexp: a = m 2^e with m in [0.5, 1)."""
    a = np.asarray(amax, dtype=np.float64)
    finite = np.isfinite(a)
    pos = finite & (a > 0)
    _, ex = np.frexp(np.where(pos, a, 1.0))
    e = ex.astype(np.int64) - 1 - EMAX_E4M3
    code = np.clip(e + E8M0_BIAS, 0, 254)
    code = np.where(pos, code, 0)
    return np.where(finite, code, E8M0_NAN).astype(np.uint8)


def quant_rows(x_bits: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """MX quantization of a bf16 [R, K] matrix along K (K % 128 == 0).

    Returns (codes uint8 [R, K], scales uint8 [K/128][R][4])."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    R, K = x_bits.shape
    assert K % 128 == 0
    x = bf16_bits_to_f32(x_bits).astype(np.float64).reshape(R, K // BLOCK, BLOCK)
    with np.errstate(invalid="ignore"):
        amax = np.max(np.abs(x), axis=2)                 # NaN propagates
    code = shared_exponent_code(amax)                    # [R, K/32]
    X = e8m0_decode(code)[:, :, None]
    with np.errstate(invalid="ignore", over="ignore"):
        v = (x / X).astype(np.float32)                   # exact: X is a power of two, |x / X| < 512
    q = e4m3.encode_nearest(v).reshape(R, K)
    xs = np.ascontiguousarray(code.reshape(R, K // 128, 4).transpose(1, 0, 2))
    return q, xs


def quant_cols(x_bits: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """MX quantization of a bf16 [T, C] matrix along T (T % 128 == 0), written transposed.

    Returns (codes uint8 [C, T], scales uint8 [T/128][C][4])."""
    return quant_rows(np.ascontiguousarray(np.asarray(x_bits, dtype=np.uint16).T))


def dequant(q: np.ndarray, xs: np.ndarray) -> np.ndarray:
    """float64 [R, K] values of MX codes and their scales."""
    R, K = q.shape
    scale = e8m0_decode(np.asarray(xs).transpose(1, 0, 2).reshape(R, K // BLOCK))
    return (e4m3.decode(q).reshape(R, K // BLOCK, BLOCK) * scale[:, :, None]).reshape(R, K)


def gemm(A: np.ndarray, xa: np.ndarray, B: np.ndarray, xb: np.ndarray, row_chunk: int = 1024) -> np.ndarray:
    """C [M, N] = dequant(A) dequant(B)^T in float64 (the exact MX product)."""
    Ad = dequant(A, xa)
    BdT = np.ascontiguousarray(dequant(B, xb).T)
    C = np.empty((Ad.shape[0], BdT.shape[1]), dtype=np.float64)
    for i in range(0, Ad.shape[0], row_chunk):
        C[i:i + row_chunk] = Ad[i:i + row_chunk] @ BdT
    return C


def operand_norms(A, xa, B, xb):
    Ad, Bd = dequant(A, xa), dequant(B, xb)
    return np.sqrt((Ad * Ad).sum(axis=1)), np.sqrt((Bd * Bd).sum(axis=1))

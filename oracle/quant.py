"""Blockwise (tile-wise) FP8 quantization, written out step by step on the CPU.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this module.

What the pages fix (no sentence quoted; restated):
  * ModelScope write-up "清华开源 Puro-2B：4400 美元训练…", section 精度 (FP8 block
    quantization): the main linear-layer matmuls run in FP8 following DeepSeek-V3's
    fine-grained block quantization; numerically sensitive work and training state
    stay in BF16/FP32.
  * agihunt digest "清华用消费级 5090 花 6890 美元从零训 2B…", section 方法 (Method),
    FP8 bullet: activations are grouped by 128, weights use 128x128 blocks.
  * same digest, section 术语 (glossary), entry "blockwise FP8": each local block
    gets its own scale so that one outlier cannot inflate a scale shared by the
    whole tensor.

Readings taken where the pages are silent (each listed in the design notes):
  * format OCP E4M3 (max 448); scale per tile s = amax / 448 in fp32, from the
    tile's own amax at call time;
  * amax is floored at 2^-96 (a zero or denormal-only tile still gets a normal,
    finite scale and reciprocal; realistic tiles are never touched);
  * the cast input is fl32(x * fl32(448 / amax_eff)): one correctly rounded fp32
    division per tile, one fp32 multiply per element;
  * the cast is saturating round-to-nearest-even (``oracle.e4m3``);
  * "grouped by 128" runs along the contraction axis of the GEMM that consumes
    the tensor: 1x128 (along features) for the forward/dgrad activation operand,
    128x1 (along tokens) for both wgrad operands;
  * NaN anywhere in a tile makes amax, the scale and every code of the tile NaN
    (NumPy's max propagates NaN); a +-Inf in a tile gives scale +Inf, code NaN for
    the infinite element and +-0 for the finite ones.  Non-finite input is
    outside the bit-exact contract.

The steps, in the order the method takes them: per tile amax -> (s, r) -> scaled
cast of every element -> emit codes and scales in the boundary's layouts.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

from .e4m3 import E4M3_MAX, encode_nearest

AMAX_FLOOR = np.float32(2.0 ** -96)
GROUP = 128


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns (uint16) to float32."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def tile_scale(amax: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Scale and reciprocal of tiles with the given (float32, non-negative) amax.

    amax_eff = max(amax, 2^-96); s = fl32(amax_eff / 448); r = fl32(448 / amax_eff),
    each one IEEE float32 operation.
    """
    amax = np.asarray(amax, dtype=np.float32)
    amax_eff = np.maximum(amax, AMAX_FLOOR)            # NaN propagates
    s = (amax_eff / np.float32(E4M3_MAX)).astype(np.float32)
    r = (np.float32(E4M3_MAX) / amax_eff).astype(np.float32)
    return s, r


def quantize_tiles(x_bits: np.ndarray, tile_rows: int, tile_cols: int) -> Tuple[np.ndarray, np.ndarray]:
    """Quantize a [R, C] bf16 tensor with one scale per (tile_rows x tile_cols) tile.

    Returns codes [R, C] (uint8, same layout as the input) and scales
    [R / tile_rows, C / tile_cols] (float32, tile-row-major).
    """
    x = bf16_bits_to_f32(x_bits)
    R, C = x.shape
    if R % tile_rows or C % tile_cols:
        raise ValueError(f"shape {x.shape} is not a multiple of the tile {tile_rows}x{tile_cols}")
    tiles = x.reshape(R // tile_rows, tile_rows, C // tile_cols, tile_cols)
    # step 1: amax of each tile
    amax = np.abs(tiles).max(axis=(1, 3))                      # [R/tr, C/tc] float32
    # step 2: scale and reciprocal of each tile
    s, r = tile_scale(amax)
    # step 3: scaled value of each element, one fp32 multiply
    with np.errstate(invalid="ignore"):
        v = (tiles * r[:, None, :, None]).astype(np.float32)
    # step 4: saturating RNE cast to E4M3
    q = encode_nearest(v).reshape(R, C)
    return q, s


def quant_act_1x128(x_bits: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """1x128 groups along the last (feature) axis of X [M, K].

    Returns codes q [M, K] and scales s [K/128, M] (contraction-block-major: the
    scales of one 128-deep slice for consecutive rows are contiguous).
    """
    q, s = quantize_tiles(x_bits, 1, GROUP)          # s: [M, K/128]
    return q, np.ascontiguousarray(s.T)


def quant_act_128x1(x_bits: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """128x1 groups along the token axis of X [T, C], output written transposed.

    Returns codes qT [C, T] (token-contiguous) and scales sT [T/128, C].
    """
    q, s = quantize_tiles(x_bits, GROUP, 1)          # q: [T, C], s: [T/128, C]
    return np.ascontiguousarray(q.T), s


def quant_w_128x128(w_bits: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """128x128 blocks of W [N, K].

    Returns q [N, K], s [N/128, K/128], and the transposed copy used by dgrad:
    qT [K, N] and sT [K/128, N/128] (the same blocks, transposed).
    """
    q, s = quantize_tiles(w_bits, GROUP, GROUP)
    return q, s, np.ascontiguousarray(q.T), np.ascontiguousarray(s.T)

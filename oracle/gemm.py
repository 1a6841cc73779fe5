"""Blockwise-scaled FP8 GEMM, as its plain definition: dequantize, then multiply.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this module.

The method (ModelScope write-up "清华开源 Puro-2B…", section 精度: the main linear
layers' matmuls run on the FP8 path, DeepSeek-V3 style; agihunt digest
"清华用消费级 5090…", section 方法, FP8 bullet: 1x128 activation groups, 128x128
weight blocks, BF16/FP32 state) accumulates each 128-deep contraction slice of
FP8 products in fp32 and adds it, multiplied by the two operands' scales of that
slice, into an fp32 accumulator.  In exact arithmetic that equals

    C[i, j] = sum_k  dec(A[i,k]) * sA(i, k/128)  *  dec(B[j,k]) * sB(j, k/128)

i.e. the product of the two dequantized operands.  This module computes exactly
that in float64: every dequantized value dec(code) * scale is exact in float64
(<= 4 significant bits times a 24-bit scale), and the float64 matmul adds
rounding of order 1e-16 relative, far below the fp32 path's own error.  The
slice-wise summation order of the GPU path is not part of the contract.

Operand layouts (all row-major, contraction axis contiguous):
  A [M, K] codes, sA [K/128, M]                               (every mode)
  FWD / DGRAD: B [N, K] codes, sB [N/128, K/128]  (128x128 weight blocks)
  WGRAD:       B [N, K] codes, sB [K/128, N]      (128x1 token groups)
"""
from __future__ import annotations

import numpy as np

from .e4m3 import decode

GROUP = 128
MODES = ("FWD", "DGRAD", "WGRAD")


def dequant_a(q: np.ndarray, s_kb_major: np.ndarray) -> np.ndarray:
    """A-operand dequantization: q [M, K], s [K/128, M] -> float64 [M, K]."""
    M, K = q.shape
    assert s_kb_major.shape == (K // GROUP, M)
    scale = np.repeat(s_kb_major.T.astype(np.float64), GROUP, axis=1)   # [M, K]
    return decode(q) * scale


def dequant_b(mode: str, q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """B-operand dequantization for the given mode -> float64 [N, K]."""
    N, K = q.shape
    if mode in ("FWD", "DGRAD"):
        assert s.shape == (N // GROUP, K // GROUP)
        scale = np.repeat(np.repeat(s.astype(np.float64), GROUP, axis=0), GROUP, axis=1)
    elif mode == "WGRAD":
        assert s.shape == (K // GROUP, N)
        scale = np.repeat(s.T.astype(np.float64), GROUP, axis=1)
    else:
        raise ValueError(mode)
    return decode(q) * scale


def gemm(mode: str, A: np.ndarray, sA: np.ndarray, B: np.ndarray, sB: np.ndarray,
         row_chunk: int = 2048) -> np.ndarray:
    """float64 C [M, N] = dequant(A) . dequant(B)^T."""
    Ad = dequant_a(A, sA)
    Bd = dequant_b(mode, B, sB)
    M = Ad.shape[0]
    C = np.empty((M, Bd.shape[0]), dtype=np.float64)
    BdT = np.ascontiguousarray(Bd.T)
    for i in range(0, M, row_chunk):
        C[i:i + row_chunk] = Ad[i:i + row_chunk] @ BdT
    return C


def gemm_rows(mode: str, A: np.ndarray, sA: np.ndarray, B: np.ndarray, sB: np.ndarray,
              rows: np.ndarray, cols: np.ndarray) -> np.ndarray:
    """float64 C[rows[t], cols[t]] for sampled output positions (full-size checks)."""
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    K = A.shape[1]
    a = decode(A[rows]) * np.repeat(sA[:, rows].T.astype(np.float64), GROUP, axis=1)
    bq = decode(B[cols])
    if mode in ("FWD", "DGRAD"):
        bs = np.repeat(sB[cols // GROUP].astype(np.float64), GROUP, axis=1)
    else:
        bs = np.repeat(sB[:, cols].T.astype(np.float64), GROUP, axis=1)
    assert a.shape == (len(rows), K)
    return np.einsum("tk,tk->t", a, bq * bs)


def operand_norms(mode: str, A, sA, B, sB):
    """Euclidean norms over the full contraction of every dequantized row of A and of B."""
    Ad = dequant_a(A, sA)
    Bd = dequant_b(mode, B, sB)
    return np.sqrt((Ad * Ad).sum(axis=1)), np.sqrt((Bd * Bd).sum(axis=1))


def bf16_round(c: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (via fp32, RNE), returned as float64.

    Used only to report the bf16 epilogue's own rounding in error budgets.
    """
    f = np.asarray(c, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)).view(np.float32)
    return r.astype(np.float64)

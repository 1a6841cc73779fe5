"""Pins of the MXFP8 oracle (oracle/mx.py) against things other than itself."""
import numpy as np
import pytest
import torch

from oracle import e4m3, mx
from oracle.quant import bf16_bits_to_f32
from workloads import f32_to_bf16_bits


def bits(x):
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def test_e8m0_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = mx.e8m0_decode(codes)
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert (got[:255] == ref[:255]).all()
    assert got[127] == 1.0 and got[0] == 2.0 ** -127 and got[254] == 2.0 ** 127


def test_shared_exponent_brute_force_every_bf16_amax():
    # floor(log2 a) by searching a table of powers of two (no frexp, no logarithm)
    a_bits = np.arange(1, 0x7F80, dtype=np.uint16)              # every finite positive bf16
    a = bf16_bits_to_f32(a_bits).astype(np.float64)
    powers = np.ldexp(1.0, np.arange(-140, 130))
    e = np.searchsorted(powers, a, side="right") - 1 - 140
    assert (np.ldexp(1.0, e) <= a).all() and (a < np.ldexp(1.0, e + 1)).all()
    expect = np.clip(e - 8 + 127, 0, 254)
    assert (mx.shared_exponent_code(a) == expect).all()
    assert mx.shared_exponent_code(np.array([0.0]))[0] == 0
    assert (mx.shared_exponent_code(np.array([np.inf, np.nan])) == 255).all()


def test_block_maximum_lands_in_256_to_512_and_error_bound():
    rng = np.random.default_rng(0)
    xb = bits(rng.standard_t(3, (64, 512)) * np.exp2(rng.integers(-40, 40, (64, 1))))
    q, xs = mx.quant_rows(xb)
    x = bf16_bits_to_f32(xb).astype(np.float64).reshape(64, 16, 32)
    X = mx.e8m0_decode(xs.transpose(1, 0, 2).reshape(64, 16))[:, :, None]
    v = x / X
    amax_v = np.abs(v).max(axis=2)
    assert ((amax_v >= 256) & (amax_v < 512)).all()
    d = e4m3.decode(q).reshape(64, 16, 32)
    dmax = np.abs(d).max(axis=2)
    assert ((dmax >= 256) & (dmax <= 448)).all()
    # half an E4M3 ulp of v (ulp 2^(floor(log2|v|) - 3), 2^-9 below the normal range), or the
    # saturation distance for |v| > 448
    av = np.abs(v)
    with np.errstate(divide="ignore"):
        ulp = np.where(av >= 2.0 ** -6, np.ldexp(1.0, np.floor(np.log2(np.where(av > 0, av, 1.0))).astype(int) - 3),
                       2.0 ** -9)
    bound = np.where(av > 448, av - 448, ulp / 2)
    assert (np.abs(v - d) <= bound * (1 + 1e-12)).all()


def test_scaled_small_integers_are_exact():
    rng = np.random.default_rng(1)
    k = rng.integers(-16, 17, (16, 256)).astype(np.float64)
    k[:, ::32] = 16                                             # every block's max is 16 * 2^p
    p = rng.integers(-60, 60, (16, 8))
    x = k * np.repeat(np.ldexp(1.0, p), 32, axis=1)
    xb = bits(x)
    assert (bf16_bits_to_f32(xb) == x).all()
    q, xs = mx.quant_rows(xb)
    assert (mx.dequant(q, xs) == x).all()
    assert (xs.transpose(1, 0, 2).reshape(16, 8) == p - 4 + 127).all()
    assert (e4m3.decode(q) == 16 * k).all()


def test_zero_tiny_and_nonfinite_blocks():
    x = np.ones((2, 128), np.float32)
    x[0, :32] = 0.0
    x[0, 32:64] = -0.0
    x[0, 64:96] = 1e-39                                          # bf16 subnormals: clamped scale
    x[1, 5] = np.nan
    x[1, 40] = np.inf
    q, xs = mx.quant_rows(bits(x))
    assert xs[0, 0, 0] == 0 and (q[0, :32] == 0).all()
    assert xs[0, 0, 1] == 0 and (q[0, 32:64] == 0x80).all()
    assert xs[0, 0, 2] == 0
    assert e4m3.decode(q[0, 64:96]).max() > 0                    # 1e-39 * 2^127 ~ 0.17: nonzero codes
    assert xs[0, 1, 0] == 255 and xs[0, 1, 1] == 255 and xs[0, 1, 2] == 127 - 8
    assert xs[0, 0, 3] == 127 - 8 and (e4m3.decode(q[0, 96:]) == 256).all()


def test_gemm_triple_loop_tiny():
    rng = np.random.default_rng(2)
    finite = np.array([c for c in range(256) if not e4m3.is_nan_code(np.uint8(c))], dtype=np.uint8)
    M, N, K = 5, 7, 256
    A = rng.choice(finite, (M, K)).astype(np.uint8)
    B = rng.choice(finite, (N, K)).astype(np.uint8)
    xa = rng.integers(110, 140, (K // 128, M, 4)).astype(np.uint8)
    xb = rng.integers(110, 140, (K // 128, N, 4)).astype(np.uint8)
    C = mx.gemm(A, xa, B, xb)
    table = e4m3.decode_table()
    for i in range(M):
        for j in range(N):
            acc = 0.0
            for k in range(K):
                sa = 2.0 ** (int(xa[k // 128, i, (k % 128) // 32]) - 127)
                sb = 2.0 ** (int(xb[k // 128, j, (k % 128) // 32]) - 127)
                acc += float(table[A[i, k]]) * sa * float(table[B[j, k]]) * sb
            assert C[i, j] == pytest.approx(acc, rel=1e-12, abs=1e-300)


def test_gemm_unit_scales_is_plain_fp8_matmul():
    rng = np.random.default_rng(3)
    A = rng.integers(0, 0x7E, (16, 128)).astype(np.uint8)
    B = rng.integers(0x80, 0xFE, (8, 128)).astype(np.uint8)
    ones = lambda r: np.full((1, r, 4), 127, np.uint8)
    C = mx.gemm(A, ones(16), B, ones(8))
    assert (C == e4m3.decode(A) @ e4m3.decode(B).T).all()


def test_cols_is_rows_of_transpose():
    rng = np.random.default_rng(4)
    xb = bits(rng.standard_normal((256, 128)))
    qT, xsT = mx.quant_cols(xb)
    q2, xs2 = mx.quant_rows(np.ascontiguousarray(xb.T))
    assert (qT == q2).all() and (xsT == xs2).all() and qT.shape == (128, 256) and xsT.shape == (2, 128, 4)

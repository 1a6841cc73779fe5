"""Pins of the oracle GEMM (CPU only).

- explicit pure-Python triple loops (a different formulation: dequantize each
  element on the fly, sum per 128-deep slice, then scale) on small shapes;
- the slice-wise promotion form sum_kb P_kb * sA * sB (exact per-slice partials)
  equals dequantize-then-matmul;
- special cases: unit scales reduce to a plain FP8 matmul; one nonzero code per
  row gives one scaled product; scaled small integers give an exact integer result;
- the bf16 rounding helper against PyTorch's own float32 -> bfloat16 conversion.
"""
import numpy as np
import pytest

from oracle import e4m3, gemm, quant
from workloads import f32_to_bf16_bits

RNG = np.random.default_rng(99)
TABLE = e4m3.decode_table()
FINITE = np.array([c for c in range(256) if not np.isnan(TABLE[c])], dtype=np.uint8)


def rand_operands(mode, M, N, K):
    A = RNG.choice(FINITE, size=(M, K))
    B = RNG.choice(FINITE, size=(N, K))
    sA = (RNG.random((K // 128, M)) * 2.0 ** RNG.integers(-20, 5, size=(K // 128, M))).astype(np.float32)
    if mode == "WGRAD":
        sB = (RNG.random((K // 128, N)) + 0.1).astype(np.float32)
    else:
        sB = (RNG.random((N // 128, K // 128)) + 0.1).astype(np.float32)
    return A, sA, B, sB


def sB_of(mode, sB, j, kb):
    return float(sB[kb, j]) if mode == "WGRAD" else float(sB[j // 128, kb])


@pytest.mark.parametrize("mode", gemm.MODES)
def test_against_explicit_loops(mode):
    M, N, K = 128, 256, 384
    A, sA, B, sB = rand_operands(mode, M, N, K)
    C = gemm.gemm(mode, A, sA, B, sB)
    for _ in range(40):
        i = int(RNG.integers(M))
        j = int(RNG.integers(N))
        total = 0.0
        mag = 0.0
        for kb in range(K // 128):
            part = 0.0
            for k in range(kb * 128, kb * 128 + 128):
                part += TABLE[A[i, k]] * TABLE[B[j, k]]
            total += part * float(sA[kb, i]) * sB_of(mode, sB, j, kb)
            mag += sum(abs(TABLE[A[i, k]] * TABLE[B[j, k]]) for k in range(kb * 128, kb * 128 + 128)) \
                * float(sA[kb, i]) * sB_of(mode, sB, j, kb)
        assert abs(C[i, j] - total) <= 1e-13 * mag, (i, j, C[i, j], total)


@pytest.mark.parametrize("mode", gemm.MODES)
def test_slice_promotion_form_equals_dequant_matmul(mode):
    M, N, K = 128, 128, 512
    A, sA, B, sB = rand_operands(mode, M, N, K)
    C = gemm.gemm(mode, A, sA, B, sB)
    acc = np.zeros((M, N))
    for kb in range(K // 128):
        sl = slice(kb * 128, kb * 128 + 128)
        P = TABLE[A[:, sl]] @ TABLE[B[:, sl]].T          # exact in float64 (< 2^43 span)
        if mode == "WGRAD":
            sc = np.outer(sA[kb].astype(np.float64), sB[kb].astype(np.float64))
        else:
            sc = np.outer(sA[kb].astype(np.float64), np.repeat(sB[:, kb].astype(np.float64), 128))
        acc += P * sc
    # float64 rounding bound relative to sum_k |A^_ik| |B^_jk| (cancellation-safe)
    mag = np.abs(gemm.dequant_a(A, sA)) @ np.abs(gemm.dequant_b(mode, B, sB)).T
    assert (np.abs(C - acc) <= 1e-13 * mag).all()


def test_unit_scales_reduce_to_plain_fp8_matmul():
    M, N, K = 128, 128, 256
    A = RNG.choice(FINITE, size=(M, K))
    B = RNG.choice(FINITE, size=(N, K))
    C = gemm.gemm("FWD", A, np.ones((2, M), np.float32), B, np.ones((1, 2), np.float32))
    # plain matmul of the decoded values in exact rational arithmetic on a few entries
    from fractions import Fraction
    for (i, j) in [(0, 0), (5, 77), (127, 127)]:
        ex = sum(Fraction(TABLE[A[i, k]]) * Fraction(TABLE[B[j, k]]) for k in range(K))
        assert C[i, j] == float(ex)


def test_one_nonzero_code_per_row_is_a_single_scaled_product():
    M, N, K = 128, 128, 256
    A = np.zeros((M, K), np.uint8)
    B = np.zeros((N, K), np.uint8)
    ka = RNG.integers(K, size=M)
    A[np.arange(M), ka] = RNG.choice(FINITE, size=M)
    B[:, :] = RNG.choice(FINITE, size=(N, K))
    sA = RNG.random((2, M)).astype(np.float32)
    sB = RNG.random((1, 2)).astype(np.float32)
    C = gemm.gemm("FWD", A, sA, B, sB)
    for i in range(0, M, 9):
        for j in range(0, N, 13):
            k = ka[i]
            ex = TABLE[A[i, k]] * float(sA[k // 128, i]) * TABLE[B[j, k]] * float(sB[0, k // 128])
            assert C[i, j] == ex


def test_scaled_small_integers_give_exact_integer_result():
    """Quantize k*2^p tiles (closed form: codes = k, s = 2^p), multiply: exact integer sums * 2^(p+q)."""
    M, N, K = 128, 128, 384
    ka = RNG.integers(-8, 9, size=(M, K)).astype(np.float64)
    kb = RNG.integers(-8, 9, size=(N, K)).astype(np.float64)
    ka[:, ::128] = 448.0
    kb[::1, 0::128] = 448.0
    pa, pb = -7, 3
    XA = f32_to_bf16_bits((ka * 2.0 ** pa).astype(np.float32))
    XB = f32_to_bf16_bits((kb * 2.0 ** pb).astype(np.float32))
    qa, sa = quant.quant_act_1x128(XA)
    qb, sb, _, _ = quant.quant_w_128x128(XB)
    assert (sa == 2.0 ** pa).all() and (sb == 2.0 ** pb).all()
    C = gemm.gemm("FWD", qa, sa, qb, sb)
    exact = (ka @ kb.T) * 2.0 ** (pa + pb)
    np.testing.assert_array_equal(C, exact)


def test_sampled_rows_match_full():
    for mode in gemm.MODES:
        A, sA, B, sB = rand_operands(mode, 256, 256, 256)
        C = gemm.gemm(mode, A, sA, B, sB)
        r = RNG.integers(256, size=50)
        c = RNG.integers(256, size=50)
        np.testing.assert_allclose(gemm.gemm_rows(mode, A, sA, B, sB, r, c), C[r, c], rtol=1e-13)


def test_bf16_round_matches_torch_rne():
    """bf16_round (used for the bit-exact bf16-output GEMM checks) against PyTorch's own
    float32 -> bfloat16 conversion (round to nearest even): random magnitudes over a wide
    range, every exact tie (low 16 bits 0x8000, both parities of the kept mantissa), and the
    integers the exact-integer GEMM tests produce."""
    import torch
    rng = np.random.default_rng(7)
    x = rng.standard_normal(200000) * np.exp2(rng.integers(-100, 100, 200000).astype(np.float64))
    hi = rng.integers(0, 1 << 16, 50000, dtype=np.uint32) & np.uint32(0x7F7F)   # finite exponents
    ties = ((hi << np.uint32(16)) | np.uint32(0x8000)).view(np.float32).astype(np.float64)
    ints = np.arange(-(1 << 15), 1 << 15, dtype=np.float64)
    for v in (x, ties, -ties, ints):
        ref = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
        got = gemm.bf16_round(v)
        assert (got == ref).all()

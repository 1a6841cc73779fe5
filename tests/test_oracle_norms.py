"""Pins of the oracle's operand norms (CPU only): the denominators of every GEMM parity bar.

The bar max |C - C_ref| / (||A^_i|| ||B^_j||) <= 1e-3 is only as strict as its
denominators, so ``gemm.operand_norms`` (blockwise scales) and ``mx.operand_norms``
(E8M0 block scales) are pinned here against things other than their own code:

- an explicit pure-Python loop in exact rational arithmetic, element by element, the
  scale of each element looked up from the layout the C ABI documents (activations
  [K/128][rows]; 128x128 weight blocks [N/128][K/128]; WGRAD per-row [K/128][N]; MX bytes
  [K/128][rows][4], byte j covering elements 32 j .. 32 j + 31 of the slice);
- a closed form: every code 0x38 (= 1.0) and power-of-two scales 2^p(row, block), so the
  squared norm is sum over blocks of (block length) * 4^p;
- a closed form: one nonzero code per row, in a block chosen per row, so the norm is
  |dec(code)| times that block's scale.

Each pin is a function of the norm routine, and the last tests plant plausible mistakes in
copies of the routine (scale axis transposed, one scale per 128x128 tile instead of per
slice, undecoded codes, MX blocks taken in the wrong byte order) and check that at least
one pin rejects each of them.
"""
from fractions import Fraction
import math

import numpy as np
import pytest

from oracle import e4m3, gemm, mx

TABLE = e4m3.decode_table()
FINITE = np.array([c for c in range(256) if not np.isnan(TABLE[c])], dtype=np.uint8)
ONE = 0x38                                     # E4M3 1.0 (OCP closed form: e = 7, m = 0)


def blockwise_scale_of(mode, operand, s, r, k):
    """Scale of element (r, k) of operand 'A' or 'B', read from the documented layouts."""
    if operand == "A":
        return float(s[k // 128, r])                       # [K/128][M]
    if mode == "WGRAD":
        return float(s[k // 128, r])                       # [K/128][N]
    return float(s[r // 128, k // 128])                    # [N/128][K/128]


def exact_norm_sq(codes, scale_of):
    """Exact squared Euclidean norm of every row: sum_k (dec(code) * scale)^2 in rationals."""
    out = []
    for r in range(codes.shape[0]):
        acc = Fraction(0)
        for k in range(codes.shape[1]):
            v = Fraction(float(TABLE[codes[r, k]])) * Fraction(scale_of(r, k))
            acc += v * v
        out.append(acc)
    return out


def close(norms, exact_sq, rel=1e-14):
    return all(abs(float(n) ** 2 - float(e)) <= rel * float(e) + 1e-300 for n, e in zip(norms, exact_sq))


# ---------------------------------------------------------------- blockwise pins

def rand_blockwise(mode, M, N, K, seed):
    rng = np.random.default_rng(seed)
    A = rng.choice(FINITE, size=(M, K)).astype(np.uint8)
    B = rng.choice(FINITE, size=(N, K)).astype(np.uint8)
    sA = (rng.random((K // 128, M)) * 2.0 ** rng.integers(-12, 6, size=(K // 128, M)) + 2.0 ** -20).astype(np.float32)
    if mode == "WGRAD":
        sB = (rng.random((K // 128, N)) * 2.0 ** rng.integers(-12, 6, size=(K // 128, N)) + 2.0 ** -20).astype(np.float32)
    else:
        sB = (rng.random((N // 128, K // 128)) * 2.0 ** rng.integers(-12, 6, size=(N // 128, K // 128))
              + 2.0 ** -20).astype(np.float32)
    return A, sA, B, sB


def pin_exact_loop(norms_fn, mode, seed=5):
    M, N, K = 6, 256, 384
    A, sA, B, sB = rand_blockwise(mode, 128, N, K, seed)
    A, sA = A[:M], np.ascontiguousarray(sA)            # keep every row's scales; only M rows are summed
    na, nb = norms_fn(mode, A, sA[:, :M], B, sB)
    ea = exact_norm_sq(A, lambda r, k: blockwise_scale_of(mode, "A", sA, r, k))
    rows_b = [0, 1, 127, 128, 200, 255]
    eb = exact_norm_sq(B[rows_b], lambda r, k: blockwise_scale_of(mode, "B", sB, rows_b[r], k))
    return close(na, ea) and close(nb[rows_b], eb)


def pin_unit_codes(norms_fn, mode):
    """Codes all 1.0; scale of (row, slice) = 2^p with p distinct per row and slice."""
    M, N, K = 256, 256, 512
    nk = K // 128
    pa = (np.arange(nk)[:, None] * 3 + np.arange(M)[None, :] % 7 - 9)             # [K/128][M]
    sA = np.exp2(pa).astype(np.float32)
    A = np.full((M, K), ONE, np.uint8)
    B = np.full((N, K), ONE, np.uint8)
    if mode == "WGRAD":
        pb = (np.arange(nk)[:, None] * 2 - np.arange(N)[None, :] % 5)               # [K/128][N]
        sB = np.exp2(pb).astype(np.float32)
        want_b = np.sqrt(128.0 * np.exp2(2.0 * pb).sum(axis=0))
    else:
        pb = (np.arange(N // 128)[:, None] * 4 - np.arange(nk)[None, :] * 2)       # [N/128][K/128]
        sB = np.exp2(pb).astype(np.float32)
        want_b = np.repeat(np.sqrt(128.0 * np.exp2(2.0 * pb).sum(axis=1)), 128)
    want_a = np.sqrt(128.0 * np.exp2(2.0 * pa).sum(axis=0))
    na, nb = norms_fn(mode, A, sA, B, sB)
    return np.allclose(na, want_a, rtol=1e-15, atol=0) and np.allclose(nb, want_b, rtol=1e-15, atol=0)


def pin_one_code_per_row(norms_fn, mode):
    """Row r holds one nonzero code c_r at column k_r; its norm is |dec(c_r)| * scale(r, k_r / 128)."""
    rng = np.random.default_rng(17)
    M, N, K = 256, 384, 640
    _, sA, _, sB = rand_blockwise(mode, M, N, K, 23)
    A = np.zeros((M, K), np.uint8)
    B = np.zeros((N, K), np.uint8)
    ka = rng.integers(0, K, size=M)
    kb = rng.integers(0, K, size=N)
    ca = rng.choice(FINITE[(FINITE & 0x7F) != 0], size=M)
    cb = rng.choice(FINITE[(FINITE & 0x7F) != 0], size=N)
    A[np.arange(M), ka] = ca
    B[np.arange(N), kb] = cb
    want_a = np.abs(TABLE[ca]) * sA[ka // 128, np.arange(M)].astype(np.float64)
    if mode == "WGRAD":
        want_b = np.abs(TABLE[cb]) * sB[kb // 128, np.arange(N)].astype(np.float64)
    else:
        want_b = np.abs(TABLE[cb]) * sB[np.arange(N) // 128, kb // 128].astype(np.float64)
    na, nb = norms_fn(mode, A, sA, B, sB)
    return np.array_equal(na, want_a) and np.array_equal(nb, want_b)


BLOCKWISE_PINS = (pin_exact_loop, pin_unit_codes, pin_one_code_per_row)


@pytest.mark.parametrize("mode", gemm.MODES)
@pytest.mark.parametrize("pin", BLOCKWISE_PINS, ids=lambda f: f.__name__)
def test_blockwise_norms_pinned(pin, mode):
    assert pin(gemm.operand_norms, mode)


def test_blockwise_norms_used_by_parity_bar_match_exact_loop_on_named_workload():
    """The tiny workload's quantized operands (what smoke() checks): exact rows of A and B."""
    from oracle import quant
    from workloads import draw
    d = draw("tiny")
    A, sA = quant.quant_act_1x128(d["X"])
    B, sB, _, _ = quant.quant_w_128x128(d["W"])
    na, nb = gemm.operand_norms("FWD", A, sA, B, sB)
    rows = [0, 77, 255]
    ea = exact_norm_sq(A[rows], lambda r, k: blockwise_scale_of("FWD", "A", sA, rows[r], k))
    eb = exact_norm_sq(B[rows], lambda r, k: blockwise_scale_of("FWD", "B", sB, rows[r], k))
    assert close(na[rows], ea) and close(nb[rows], eb)


# planted mistakes (copies of the routine with one error each; the oracle itself is untouched)

def mutant_a_scale_axis(mode, A, sA, B, sB):
    """sA [K/128][M] read as if it were [M][K/128] (a row-major misread of the same array)."""
    M, K = A.shape
    Ad = e4m3.decode(A) * np.repeat(sA.reshape(M, K // 128).astype(np.float64), 128, axis=1)
    Bd = gemm.dequant_b(mode, B, sB)
    return np.sqrt((Ad * Ad).sum(axis=1)), np.sqrt((Bd * Bd).sum(axis=1))


def mutant_b_layout_misread(mode, A, sA, B, sB):
    """B's scale array read in the other mode's order: WGRAD [K/128][N] as [N][K/128]; FWD /
    DGRAD [N/128][K/128] as [K/128][N/128]."""
    Ad = gemm.dequant_a(A, sA)
    N, K = B.shape
    if mode == "WGRAD":
        sc = np.repeat(sB.reshape(N, K // 128).astype(np.float64), 128, axis=1)
    else:
        t = sB.reshape(K // 128, N // 128).T
        sc = np.repeat(np.repeat(t.astype(np.float64), 128, axis=0), 128, axis=1)
    Bd = e4m3.decode(B) * sc
    return np.sqrt((Ad * Ad).sum(axis=1)), np.sqrt((Bd * Bd).sum(axis=1))


def mutant_b_per_tile(mode, A, sA, B, sB):
    """One scale per row or block for the whole contraction (slice 0's), not one per slice."""
    Ad = gemm.dequant_a(A, sA)
    if mode == "WGRAD":
        Bd = e4m3.decode(B) * sB[0].astype(np.float64)[:, None]
    else:
        Bd = e4m3.decode(B) * np.repeat(sB[:, :1].astype(np.float64), 128, axis=0)
    return np.sqrt((Ad * Ad).sum(axis=1)), np.sqrt((Bd * Bd).sum(axis=1))


def mutant_undecoded(mode, A, sA, B, sB):
    Ad = A.astype(np.float64) * np.repeat(sA.T.astype(np.float64), 128, axis=1)
    Bd = gemm.dequant_b(mode, B, sB)
    return np.sqrt((Ad * Ad).sum(axis=1)), np.sqrt((Bd * Bd).sum(axis=1))


def mutant_l1(mode, A, sA, B, sB):
    Ad, Bd = gemm.dequant_a(A, sA), gemm.dequant_b(mode, B, sB)
    return np.abs(Ad).sum(axis=1), np.abs(Bd).sum(axis=1)


def _rejected(mutant, mode):
    for pin in BLOCKWISE_PINS:
        try:
            if not pin(mutant, mode):
                return True
        except (ValueError, IndexError, AssertionError):
            return True
    return False


@pytest.mark.parametrize("mode", gemm.MODES)
@pytest.mark.parametrize("mutant", (mutant_a_scale_axis, mutant_b_layout_misread, mutant_b_per_tile,
                                    mutant_undecoded, mutant_l1), ids=lambda f: f.__name__)
def test_blockwise_pins_reject_planted_mistakes(mutant, mode):
    assert _rejected(mutant, mode), f"{mutant.__name__} passes every pin in {mode}"


# ---------------------------------------------------------------- MX pins

def mx_exact_loop(norms_fn, seed=3):
    rng = np.random.default_rng(seed)
    R, K = 5, 256
    A = rng.choice(FINITE, size=(R, K)).astype(np.uint8)
    B = rng.choice(FINITE, size=(R + 2, K)).astype(np.uint8)
    xa = rng.integers(100, 150, size=(K // 128, R, 4)).astype(np.uint8)
    xb = rng.integers(100, 150, size=(K // 128, R + 2, 4)).astype(np.uint8)
    na, nb = norms_fn(A, xa, B, xb)
    sc = lambda x: (lambda r, k: math.ldexp(1.0, int(x[k // 128, r, (k % 128) // 32]) - 127))
    return close(na, exact_norm_sq(A, sc(xa))) and close(nb, exact_norm_sq(B, sc(xb)))


def mx_unit_codes(norms_fn):
    R, K = 64, 512
    A = np.full((R, K), ONE, np.uint8)
    p = (np.arange(K // 128)[:, None, None] * 4 + np.arange(4)[None, None, :] - np.arange(R)[None, :, None] % 3)
    xa = (p + 127).astype(np.uint8)                                   # [K/128][R][4]
    want = np.sqrt(32.0 * np.exp2(2.0 * p).sum(axis=(0, 2)))
    na, nb = norms_fn(A, xa, A, xa)
    return np.allclose(na, want, rtol=1e-15, atol=0) and np.allclose(nb, want, rtol=1e-15, atol=0)


def mx_one_code_per_row(norms_fn):
    rng = np.random.default_rng(29)
    R, K = 96, 384
    A = np.zeros((R, K), np.uint8)
    k = rng.integers(0, K, size=R)
    c = rng.choice(FINITE[(FINITE & 0x7F) != 0], size=R)
    A[np.arange(R), k] = c
    xa = rng.integers(90, 160, size=(K // 128, R, 4)).astype(np.uint8)
    want = np.abs(TABLE[c]) * np.exp2(xa[k // 128, np.arange(R), (k % 128) // 32].astype(np.float64) - 127)
    na, nb = norms_fn(A, xa, A, xa)
    return np.array_equal(na, want) and np.array_equal(nb, want)


MX_PINS = (mx_exact_loop, mx_unit_codes, mx_one_code_per_row)


@pytest.mark.parametrize("pin", MX_PINS, ids=lambda f: f.__name__)
def test_mx_norms_pinned(pin):
    assert pin(mx.operand_norms)


def mx_mutant_byte_order(A, xa, B, xb):
    """Scale bytes read as [rows][K/128][4] instead of [K/128][rows][4]."""
    def dq(q, x):
        R, K = q.shape
        sc = mx.e8m0_decode(np.asarray(x).reshape(R, K // 32))
        return (e4m3.decode(q).reshape(R, K // 32, 32) * sc[:, :, None]).reshape(R, K)
    Ad, Bd = dq(A, xa), dq(B, xb)
    return np.sqrt((Ad * Ad).sum(axis=1)), np.sqrt((Bd * Bd).sum(axis=1))


def mx_mutant_block_reversed(A, xa, B, xb):
    """The four bytes of a slice applied in reverse order."""
    return mx.operand_norms(A, xa[:, :, ::-1].copy(), B, xb[:, :, ::-1].copy())


def mx_mutant_undecoded(A, xa, B, xb):
    def dq(q, x):
        R, K = q.shape
        sc = mx.e8m0_decode(np.asarray(x).transpose(1, 0, 2).reshape(R, K // 32))
        return (q.astype(np.float64).reshape(R, K // 32, 32) * sc[:, :, None]).reshape(R, K)
    Ad, Bd = dq(A, xa), dq(B, xb)
    return np.sqrt((Ad * Ad).sum(axis=1)), np.sqrt((Bd * Bd).sum(axis=1))


@pytest.mark.parametrize("mutant", (mx_mutant_byte_order, mx_mutant_block_reversed, mx_mutant_undecoded),
                         ids=lambda f: f.__name__)
def test_mx_pins_reject_planted_mistakes(mutant):
    rejected = False
    for pin in MX_PINS:
        try:
            rejected |= not pin(mutant)
        except (ValueError, IndexError):
            rejected = True
    assert rejected, f"{mutant.__name__} passes every MX pin"

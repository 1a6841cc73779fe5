"""GPU parity past 2^31 elements: every kernel on a tensor with more than 2^31 elements (byte
offsets beyond 2^32 for bf16), so that any 32-bit row, column, scale or byte index inside a
kernel would land on the wrong element.  Checked against the oracle on sampled rows / token
blocks on both sides of the 2^31 boundary and at the very end.

Sizes: activations [262272, 8192] bf16 (2049 token blocks, 2^31 + 2^20 elements, 4.3 GB), a
weight [65664, 32768] (2^31 + 2^22 elements), a FWD output [262272, 8192] bf16 and a WGRAD-
style contraction of K = 1114112 (A [2048, K]: 2.3 GB of codes, row offsets past 2^31).
Inputs are drawn on the GPU by torch's seeded generator in row chunks; only sampled rows
travel to the host.  Bars as for the full-size tests: quantizers byte-identical, GEMMs within
1e-3 of the normalized bound (plus bf16 rounding for bf16 outputs).
"""
import numpy as np
import pytest

from gpu_util import assert_bytes_equal, host, normalized_error, say, torch
from oracle import gemm, mx, quant

pytestmark = pytest.mark.gpu

BIG_T = 262272          # 2049 blocks of 128 tokens: BIG_T * 8192 = 2^31 + 2^20
C8K = 8192
BOUNDARY_ROW = (1 << 31) // C8K     # first row whose elements lie past 2^31 (262144)
TOL = 1e-3


@pytest.fixture(scope="module")
def P():
    import blockwise_scaled_fp8_quant_amd as P
    assert torch().cuda.is_available(), "GPU test run without a GPU"
    return P


def gen(seed):
    g = torch().Generator(device="cuda")
    g.manual_seed(seed)
    return g


def normal_bf16(shape, seed, scale=1.0, chunk=16384):
    """N(0, scale^2) in bf16, drawn in row chunks (no full-size fp32 temporary)."""
    t = torch()
    x = t.empty(shape, dtype=t.bfloat16, device="cuda")
    g = gen(seed)
    for r in range(0, shape[0], chunk):
        n = min(chunk, shape[0] - r)
        x[r:r + n] = (t.randn((n, shape[1]), generator=g, device="cuda") * scale).to(t.bfloat16)
    return x


def random_codes(shape, seed):
    """Uniform E4M3 codes without NaN (magnitude codes 0x00..0x7E, random sign), drawn in row
    chunks of about 2^26 elements."""
    t = torch()
    q = t.empty(shape, dtype=t.uint8, device="cuda")
    g = gen(seed)
    chunk = max(1, (1 << 26) // shape[1])
    for r in range(0, shape[0], chunk):
        n = min(chunk, shape[0] - r)
        mag = t.randint(0, 0x7F, (n, shape[1]), generator=g, device="cuda", dtype=t.uint8)
        sign = t.randint(0, 2, (n, shape[1]), generator=g, device="cuda", dtype=t.uint8) << 7
        q[r:r + n] = mag | sign
    return q


def log_uniform(shape, seed, lo=-14, hi=-2):
    t = torch()
    return t.exp2(t.rand(shape, generator=gen(seed), device="cuda") * (hi - lo) + lo)


def bits_of(x_rows):
    t = torch()
    return x_rows.contiguous().view(t.int16).cpu().numpy().view(np.uint16)


def free():
    t = torch()
    t.cuda.synchronize()
    t.cuda.empty_cache()


@pytest.fixture(scope="module")
def big_x():
    say(f"[large] drawing x [{BIG_T}, {C8K}] bf16 ({BIG_T * C8K / 2 ** 31:.4f} x 2^31 elements)")
    x = normal_bf16((BIG_T, C8K), 7, scale=3.0)
    yield x
    del x
    free()


ROWS = [0, 131071, BOUNDARY_ROW - 1, BOUNDARY_ROW, BOUNDARY_ROW + 77, BIG_T - 1]
BLOCKS = [0, BOUNDARY_ROW // 128 - 1, BOUNDARY_ROW // 128]     # the last block starts at 2^31


def test_quant_1x128_past_2g_elements(P, big_x):
    t = torch()
    say("[large] quant_act_1x128")
    q, s = P.puro_fp8_quant_act_1x128(big_x)
    t.cuda.synchronize()
    rows = t.tensor(ROWS, device="cuda")
    rq, rs = quant.quant_act_1x128(bits_of(big_x[rows]))
    assert_bytes_equal(host(q[rows]), rq, "1x128 codes of sampled rows")
    assert_bytes_equal(host(s[:, rows]), rs, "1x128 scales of sampled rows")
    del q, s
    free()


def test_quant_128x1_past_2g_elements(P, big_x):
    t = torch()
    say("[large] quant_act_128x1")
    qT, sT = P.puro_fp8_quant_act_128x1(big_x)
    t.cuda.synchronize()
    for tb in BLOCKS:
        rows = slice(128 * tb, 128 * tb + 128)
        rqT, rsT = quant.quant_act_128x1(bits_of(big_x[rows]))
        assert_bytes_equal(host(qT[:, rows]), rqT, f"128x1 codes of token block {tb}")
        assert_bytes_equal(host(sT[tb:tb + 1]), rsT, f"128x1 scales of token block {tb}")
    del qT, sT
    free()


def test_dual_past_2g_elements(P, big_x):
    t = torch()
    say("[large] quant_act_dual")
    q, s, qT, sT = P.puro_fp8_quant_act_dual(big_x)
    t.cuda.synchronize()
    for tb in BLOCKS:
        rows = slice(128 * tb, 128 * tb + 128)
        xb = bits_of(big_x[rows])
        rq, rs = quant.quant_act_1x128(xb)
        rqT, rsT = quant.quant_act_128x1(xb)
        assert_bytes_equal(host(q[rows]), rq, f"dual row codes of token block {tb}")
        assert_bytes_equal(host(s[:, rows]), rs, f"dual row scales of token block {tb}")
        assert_bytes_equal(host(qT[:, rows]), rqT, f"dual transposed codes of token block {tb}")
        assert_bytes_equal(host(sT[tb:tb + 1]), rsT, f"dual column scales of token block {tb}")
    del q, s, qT, sT
    free()


def test_mx_dual_past_2g_elements(P, big_x):
    t = torch()
    say("[large] mx_quant_dual")
    q, xs, qT, xsT = P.puro_fp8_mx_quant_dual(big_x)
    t.cuda.synchronize()
    for tb in BLOCKS:
        rows = slice(128 * tb, 128 * tb + 128)
        xb = bits_of(big_x[rows])
        rq, rxs = mx.quant_rows(xb)
        rqT, rxsT = mx.quant_cols(xb)
        assert_bytes_equal(host(q[rows]), rq, f"MX row codes of token block {tb}")
        assert_bytes_equal(host(xs[:, rows]), rxs, f"MX row scales of token block {tb}")
        assert_bytes_equal(host(qT[:, rows]), rqT, f"MX transposed codes of token block {tb}")
        assert_bytes_equal(host(xsT[tb:tb + 1]), rxsT, f"MX column scales of token block {tb}")
    del q, xs, qT, xsT
    free()


def test_quant_w_past_2g_elements(P):
    t = torch()
    N, K = 65664, 32768                      # 513 x 256 blocks: 2^31 + 2^22 elements
    say(f"[large] quant_w_128x128 [{N}, {K}]")
    w = normal_bf16((N, K), 11, scale=0.02, chunk=4096)
    q, s, qT, sT = P.puro_fp8_quant_w_128x128(w)
    t.cuda.synchronize()
    for rb in (0, (1 << 31) // K // 128 - 1, N // 128 - 1):
        rows = slice(128 * rb, 128 * rb + 128)
        rq, rs, rqT, rsT = quant.quant_w_128x128(bits_of(w[rows]))
        assert_bytes_equal(host(q[rows]), rq, f"weight codes of block row {rb}")
        assert_bytes_equal(host(s[rb:rb + 1]), rs, f"weight scales of block row {rb}")
        assert_bytes_equal(host(qT[:, rows]), rqT, f"transposed weight codes of block row {rb}")
        assert_bytes_equal(host(sT[:, rb:rb + 1]), rsT, f"transposed weight scales of block row {rb}")
    del w, q, s, qT, sT
    free()


def check_rows(Ad, Bd, sub, bf16_out):
    ref = Ad @ Bd.T
    na, nb = np.sqrt((Ad * Ad).sum(1)), np.sqrt((Bd * Bd).sum(1))
    err, diff, den = normalized_error(sub, ref, na, nb)
    say(f"    max normalized error {err:.3e} (bf16 output rounding included)")
    rnd = 2.0 ** -8 * np.abs(ref) * (1 + 2.0 ** -7) if bf16_out else 0.0
    assert (diff <= TOL * den + rnd).all()


def test_gemm_fwd_output_past_2g_elements(P):
    t = torch()
    M, N, K = BIG_T, C8K, 256
    say(f"[large] FWD GEMM {M}x{N}x{K}, bf16 output of {M * N / 2 ** 31:.4f} x 2^31 elements")
    A, B = random_codes((M, K), 21), random_codes((N, K), 22)
    sA, sB = log_uniform((K // 128, M), 23), log_uniform((N // 128, K // 128), 24)
    C = P.puro_fp8_gemm(P.FWD, A, sA, B, sB, out_dtype=P.OUT_BF16)
    t.cuda.synchronize()
    rows = t.tensor(ROWS, device="cuda")
    Ad = gemm.dequant_a(host(A[rows]), host(sA[:, rows]))
    Bd = gemm.dequant_b("FWD", host(B), host(sB))
    check_rows(Ad, Bd, host(C[rows]), True)
    del A, B, sA, sB, C
    free()


def test_mx_gemm_output_past_2g_elements(P):
    t = torch()
    M, N, K = BIG_T, C8K, 256
    say(f"[large] MX GEMM {M}x{N}x{K}, bf16 output")
    A, B = random_codes((M, K), 31), random_codes((N, K), 32)
    xa = t.randint(115, 136, (K // 128, M, 4), generator=gen(33), device="cuda", dtype=t.uint8)
    xb = t.randint(115, 136, (K // 128, N, 4), generator=gen(34), device="cuda", dtype=t.uint8)
    C = P.puro_fp8_mx_gemm(A, xa, B, xb, out_dtype=P.OUT_BF16)
    t.cuda.synchronize()
    rows = t.tensor(ROWS, device="cuda")
    Ad = mx.dequant(host(A[rows]), host(xa[:, rows]))
    Bd = mx.dequant(host(B), host(xb))
    check_rows(Ad, Bd, host(C[rows]), True)
    del A, B, xa, xb, C
    free()


def test_gemm_wgrad_contraction_past_2g_bytes(P):
    """A [2048, K] with K = 1114112: row 2047 starts 2.28e9 bytes in (past 2^31); the contraction
    is split over K, so the split partials and their reduce run at this size too."""
    t = torch()
    M, N, K = 2048, 256, 1114112
    say(f"[large] WGRAD GEMM {M}x{N}x{K} (A: {M * K / 2 ** 31:.3f} x 2^31 bytes)")
    A, B = random_codes((M, K), 41), random_codes((N, K), 42)
    sA, sB = log_uniform((K // 128, M), 43), log_uniform((K // 128, N), 44)
    C = P.puro_fp8_gemm(P.WGRAD, A, sA, B, sB, out_dtype=P.OUT_FP32)
    t.cuda.synchronize()
    rows = np.array([0, 1023, 2046, 2047])
    rt = t.from_numpy(rows).cuda()
    Ah, sAh, Bh, sBh = host(A[rt]), host(sA[:, rt]), host(B), host(sB)
    # the oracle's dequantize-then-matmul over 128-aligned pieces of K (sums in float64)
    ref = np.zeros((len(rows), N))
    na2, nb2 = np.zeros(len(rows)), np.zeros(N)
    step = 131072
    for k0 in range(0, K, step):
        k1 = min(K, k0 + step)
        Ad = gemm.dequant_a(Ah[:, k0:k1], sAh[k0 // 128:k1 // 128])
        Bd = gemm.dequant_b("WGRAD", Bh[:, k0:k1], sBh[k0 // 128:k1 // 128])
        ref += Ad @ Bd.T
        na2 += (Ad * Ad).sum(1)
        nb2 += (Bd * Bd).sum(1)
    err, diff, den = normalized_error(host(C[rt]), ref, np.sqrt(na2), np.sqrt(nb2))
    say(f"    max normalized error {err:.3e}")
    assert err <= TOL
    del A, B, sA, sB, C
    free()

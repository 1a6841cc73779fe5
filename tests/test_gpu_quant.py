"""GPU parity of the three quantizers and the device cast against the oracle (bit-exact).

Bar: codes and fp32 scales byte-identical to the oracle on the same bf16 inputs.
Non-finite inputs are outside the bit-exact contract; their reading (NaN tile ->
NaN scale and NaN codes; inf -> scale +inf, NaN code at the inf) is checked as such.
"""
import numpy as np
import pytest

from gpu_util import assert_bytes_equal, bf16_dev, f32_dev, host, say, torch
from oracle import e4m3, quant
from workloads import draw, f32_to_bf16_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P():
    import blockwise_scaled_fp8_quant_amd as P
    t = torch()
    assert t.cuda.is_available(), "GPU test run without a GPU"
    return P


def bf16(x):
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def run_1x128(P, bits, ldx_pad=0, ldq_pad=0):
    t = torch()
    M, K = bits.shape
    xd = bf16_dev(np.pad(bits, ((0, 0), (0, ldx_pad)))) if ldx_pad else bf16_dev(bits)
    x = xd[:, :K] if ldx_pad else xd
    qbuf = t.full((M, K + ldq_pad), 0xA5, dtype=t.uint8, device="cuda")
    s = t.full((K // 128, M), float("nan"), dtype=t.float32, device="cuda")
    P.puro_fp8_quant_act_1x128(x, qbuf[:, :K], s)
    qh = host(qbuf)
    if ldq_pad:
        assert (qh[:, K:] == 0xA5).all(), "write outside the row"
    return qh[:, :K], host(s)


def check_1x128(P, bits, what, **kw):
    say(f"[quant 1x128] {what} shape={bits.shape} {kw}")
    q, s = run_1x128(P, bits, **kw)
    rq, rs = quant.quant_act_1x128(bits)
    assert_bytes_equal(s, rs, f"{what} scales")
    assert_bytes_equal(q, rq, f"{what} codes")


def check_128x1(P, bits, what, ldqT_pad=0):
    t = torch()
    say(f"[quant 128x1] {what} shape={bits.shape}")
    T, C = bits.shape
    qbuf = t.full((C, T + ldqT_pad), 0xA5, dtype=t.uint8, device="cuda")
    sT = t.full((T // 128, C), float("nan"), dtype=t.float32, device="cuda")
    P.puro_fp8_quant_act_128x1(bf16_dev(bits), qbuf[:, :T], sT)
    qh = host(qbuf)
    if ldqT_pad:
        assert (qh[:, T:] == 0xA5).all()
    rq, rs = quant.quant_act_128x1(bits)
    assert_bytes_equal(host(sT), rs, f"{what} scales")
    assert_bytes_equal(qh[:, :T], rq, f"{what} codes")


def check_w(P, bits, what, transposed=True):
    say(f"[quant 128x128] {what} shape={bits.shape} transposed={transposed}")
    q, s, qT, sT = P.puro_fp8_quant_w_128x128(bf16_dev(bits), transposed=transposed)
    rq, rs, rqT, rsT = quant.quant_w_128x128(bits)
    assert_bytes_equal(host(s), rs, f"{what} scales")
    assert_bytes_equal(host(q), rq, f"{what} codes")
    if transposed:
        assert_bytes_equal(host(sT), rsT, f"{what} scales^T")
        assert_bytes_equal(host(qT), rqT, f"{what} codes^T")


# --------------------------------------------------------------------------- device cast

def test_cast_exhaustive_all_fp32_patterns(P):
    """All 2^32 fp32 bit patterns through the device cast.

    The cast's result is a function of (sign, exponent, mantissa bits 22..19, any of bits
    18..0 set); that reduction is pinned on the oracle (test_reduction_key_is_sufficient).
    The oracle encodes one representative per key (2^14 keys), and every GPU code is
    compared with its key's oracle code; NaN inputs must give a NaN code.
    """
    t = torch()
    keys = np.arange(1 << 14, dtype=np.uint32)
    reps = ((keys >> np.uint32(1)) << np.uint32(19)) | (keys & np.uint32(1))
    table = e4m3.encode_nearest(reps.view(np.float32))
    table_d = t.from_numpy(table).to("cuda")
    chunk = 1 << 28
    for start in range(0, 1 << 32, chunk):
        say(f"[cast] chunk {start:#x}")
        u = t.arange(start, start + chunk, dtype=t.int64, device="cuda")
        v = u.to(t.int32).view(t.float32)                     # wraps to the same 32-bit pattern
        q = P.puro_fp8_cast_e4m3(v)
        key = ((u >> 19) << 1) | ((u & 0x7FFFF) != 0).to(t.int64)
        exp = table_d[key]
        nan = t.isnan(v)
        bad_finite = ((q != exp) & ~nan).sum().item()
        bad_nan = (((q & 0x7F) != 0x7F) & nan).sum().item()
        assert bad_finite == 0 and bad_nan == 0, (hex(start), bad_finite, bad_nan)
        del u, v, q, key, exp, nan


def test_cast_named_values(P):
    vals = np.array([0.0, -0.0, 1.0, -1.0, 448.0, 448.0 * (1 + 2 ** -23), 460.0, 464.0, 480.0, 1e30, np.inf,
                     -np.inf, 2.0 ** -10, 3 * 2.0 ** -10, -2.0 ** -11, 1e-40, -1e-40, 2.0 ** -9, 0.875 * 2.0 ** -6,
                     1.0 + 1 / 16, 1.0 + 3 / 16, 17.0, 18.0, 19.0], dtype=np.float32)
    q = host(P.puro_fp8_cast_e4m3(f32_dev(vals)))
    np.testing.assert_array_equal(q, e4m3.encode_nearest(vals))
    assert e4m3.is_nan_code(host(P.puro_fp8_cast_e4m3(f32_dev(np.array([np.nan] * 4, np.float32))))).all()


def test_cast_ragged_lengths(P):
    rng = np.random.default_rng(5)
    for n in (1, 2, 3, 5, 7, 1000, 4099):
        v = (rng.standard_normal(n) * 50).astype(np.float32)
        q = host(P.puro_fp8_cast_e4m3(f32_dev(v)))
        np.testing.assert_array_equal(q, e4m3.encode_nearest(v))


# --------------------------------------------------------------------------- 1x128

def test_1x128_tiny_workload(P):
    check_1x128(P, draw("tiny")["X"], "tiny X")


@pytest.mark.parametrize("name,tensor", [("qkv_fwd", "X"), ("mlp_fwd", "X"), ("mlp_fwd", "H"), ("down_bwd", "dY")])
def test_1x128_workloads(P, name, tensor):
    check_1x128(P, draw(name)[tensor], f"{name}.{tensor}")


@pytest.mark.parametrize("M,K", [(1, 128), (3, 256), (17, 384), (129, 640), (1000, 128), (33, 1536)])
def test_1x128_ragged_rows(P, M, K):
    rng = np.random.default_rng(M * 7 + K)
    check_1x128(P, bf16(rng.standard_normal((M, K)) * 3), f"ragged {M}x{K}")


def test_1x128_strided(P):
    rng = np.random.default_rng(11)
    check_1x128(P, bf16(rng.standard_t(3, (70, 512))), "strided", ldx_pad=24, ldq_pad=48)


def test_1x128_every_bf16_amax(P):
    """One row per finite non-negative bf16 amax value (32640 rows): scales and codes exact.

    Row m has amax = bf16 pattern m at a varying position, the other elements are
    bf16 values with |x| <= amax spread over [0, amax].
    """
    rng = np.random.default_rng(3)
    amax_bits = np.arange(0x7F80, dtype=np.uint16)
    amax = quant.bf16_bits_to_f32(amax_bits).astype(np.float64)
    frac = rng.random((len(amax_bits), 128))
    sign = np.where(rng.random((len(amax_bits), 128)) < 0.5, -1.0, 1.0)
    x = (sign * frac * amax[:, None]).astype(np.float32)
    xb = f32_to_bf16_bits(x)
    # bf16 rounding may round up past amax: clamp magnitudes to the amax bits (same sign)
    mag = np.minimum(xb & np.uint16(0x7FFF), amax_bits[:, None])
    xb = (xb & np.uint16(0x8000)) | mag
    pos = rng.integers(0, 128, size=len(amax_bits))
    xb[np.arange(len(amax_bits)), pos] = amax_bits
    check_1x128(P, xb.astype(np.uint16), "every bf16 amax")


def test_1x128_zero_denormal_and_huge_tiles(P):
    x = np.zeros((6, 256), np.float32)
    x[1, :] = -0.0
    x[2, :128] = 1e-39          # bf16 denormals
    x[2, 128:] = -3e-39
    x[3, :] = 3.3e38            # near the bf16 maximum
    x[3, 5] = -3.38e38
    x[4, :] = 2.0 ** -96        # exactly the amax floor
    x[5, :] = np.linspace(-1e-30, 1e-30, 256)
    check_1x128(P, bf16(x), "zero/denormal/huge")


def test_1x128_nonfinite_reading(P):
    x = np.ones((4, 256), np.float32)
    x[0, 3] = np.nan
    x[1, 4] = np.inf
    x[2, 130] = -np.inf
    q, s = run_1x128(P, bf16(x))
    assert np.isnan(s[0, 0]) and e4m3.is_nan_code(q[0, :128]).all()
    assert s[0, 1] == np.inf and s[1, 2] == np.inf
    assert e4m3.is_nan_code(q[1, 4]) and e4m3.is_nan_code(q[2, 130])
    assert (q[1, :128][np.arange(128) != 4] == 0).all()
    rq, rs = quant.quant_act_1x128(bf16(x))
    assert_bytes_equal(s[:, 3], rs[:, 3], "finite row scales")
    assert_bytes_equal(q[3], rq[3], "finite row codes")


def test_1x128_deterministic(P):
    bits = draw("qkv_fwd")["X"]
    a = run_1x128(P, bits)
    b = run_1x128(P, bits)
    assert_bytes_equal(a[0], b[0], "repeat codes")
    assert_bytes_equal(a[1], b[1], "repeat scales")


# --------------------------------------------------------------------------- 128x1

@pytest.mark.parametrize("name,tensor", [("down_bwd", "dY"), ("down_bwd", "H"), ("tiny", "X")])
def test_128x1_workloads(P, name, tensor):
    check_128x1(P, draw(name)[tensor], f"{name}.{tensor}")


@pytest.mark.parametrize("T,C", [(128, 8), (128, 72), (256, 200), (384, 64), (128, 1000)])
def test_128x1_ragged_columns(P, T, C):
    rng = np.random.default_rng(T + C)
    check_128x1(P, bf16(rng.standard_t(3, (T, C)) * 0.01), f"ragged {T}x{C}", ldqT_pad=16)


def test_128x1_is_transpose_of_1x128(P):
    rng = np.random.default_rng(21)
    bits = bf16(rng.standard_normal((512, 384)))
    t = torch()
    qT, sT = P.puro_fp8_quant_act_128x1(bf16_dev(bits))
    q2, s2 = P.puro_fp8_quant_act_1x128(bf16_dev(np.ascontiguousarray(bits.T)))
    assert_bytes_equal(host(qT), host(q2), "codes")
    assert_bytes_equal(host(sT), host(s2), "scales")


def test_128x1_zero_and_outlier_columns(P):
    x = np.zeros((256, 128), np.float32)
    x[:, 1] = -0.0
    x[7, 2] = 1e4
    x[:, 3] = 1e-39
    x[200, 4] = -2.5
    check_128x1(P, bf16(x), "zero/outlier columns")


# --------------------------------------------------------------------------- 128x128

def test_w_tiny(P):
    check_w(P, draw("tiny")["W"], "tiny W")


@pytest.mark.parametrize("name,tensor", [("qkv_fwd", "W"), ("mlp_fwd", "W_gu"), ("mlp_fwd", "W_d")])
def test_w_workloads(P, name, tensor):
    check_w(P, draw(name)[tensor], f"{name}.{tensor}")


def test_w_without_transposed_copy(P):
    rng = np.random.default_rng(8)
    check_w(P, bf16(rng.standard_normal((256, 384)) * 0.02), "no qT", transposed=False)


def test_w_outlier_isolation_and_extremes(P):
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((384, 256)) * 0.02).astype(np.float32)
    x[130, 200] = 50.0
    x[0:128, 0:128] = 0.0
    x[256:384, 128:256] *= 1e-35
    check_w(P, bf16(x), "outlier/zero/tiny blocks")


def test_w_transposed_codes_every_byte_value(P):
    """Values spread so that a block's codes take (nearly) every E4M3 byte in every position of a
    thread's 8 x 8 sub-block: the transposed copy must be the byte transpose of the row codes
    (the kernel builds it from them with byte permutes) and equal the oracle's."""
    rng = np.random.default_rng(31)
    mags = 2.0 ** rng.uniform(-9.0, 8.8, (256, 512))
    x = (np.where(rng.random((256, 512)) < 0.5, -1.0, 1.0) * mags).astype(np.float32)
    x[0:128, 0:128] *= 1e-3                              # a second block scale
    bits = bf16(x)
    q, s, qT, sT = P.puro_fp8_quant_w_128x128(bf16_dev(bits), transposed=True)
    q, qT = host(q), host(qT)
    assert len(np.unique(q[128:256, 128:256])) > 200, "the probe should cover most code bytes"
    assert_bytes_equal(qT, np.ascontiguousarray(q.T), "codes^T vs transpose of codes")
    check_w(P, bits, "every byte value")


def test_w_nonfinite_reading(P):
    """A NaN in a block gives a NaN scale and NaN codes for the whole block; an inf gives scale +inf
    and a NaN code at the inf (zero elsewhere).  The transposed copy holds the same bytes."""
    x = np.ones((256, 384), np.float32) * 0.5
    x[3, 5] = np.nan                                      # block (0, 0)
    x[140, 300] = np.inf                                  # block (1, 2)
    bits = bf16(x)
    q, s, qT, sT = P.puro_fp8_quant_w_128x128(bf16_dev(bits), transposed=True)
    q, s, qT, sT = host(q), host(s), host(qT), host(sT)
    assert np.isnan(s[0, 0]) and e4m3.is_nan_code(q[:128, :128]).all()
    assert s[1, 2] == np.inf and e4m3.is_nan_code(q[140, 300])
    blk = q[128:256, 256:384].copy()
    blk[12, 44] = 0
    assert (blk == 0).all()
    assert_bytes_equal(qT, np.ascontiguousarray(q.T), "codes^T vs transpose of codes")
    assert_bytes_equal(sT, np.ascontiguousarray(s.T), "scales^T vs transpose of scales")
    rq, rs, _, _ = quant.quant_w_128x128(bits)
    for bi, bj in ((0, 1), (0, 2), (1, 0), (1, 1)):       # the finite blocks
        assert_bytes_equal(q[128 * bi:128 * bi + 128, 128 * bj:128 * bj + 128],
                           rq[128 * bi:128 * bi + 128, 128 * bj:128 * bj + 128], f"finite block {bi},{bj}")
        assert_bytes_equal(s[bi, bj], rs[bi, bj], f"finite block scale {bi},{bj}")

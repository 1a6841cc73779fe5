"""GPU parity of the dual quantizer (one read -> 1x128 row codes + 128x1 transposed codes).

Bar: all four outputs byte-identical to the oracle's quant_act_1x128 and quant_act_128x1
on the same bf16 input.  Non-finite inputs follow the same reading as the single
quantizers (NaN -> NaN codes and a NaN scale for every tile containing it; inf -> scale +inf).
"""
import numpy as np
import pytest

from gpu_util import assert_bytes_equal, bf16_dev, host, say, torch
from oracle import e4m3, quant
from workloads import draw, f32_to_bf16_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P():
    import blockwise_scaled_fp8_quant_amd as P
    assert torch().cuda.is_available(), "GPU test run without a GPU"
    return P


def bf16(x):
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def run_dual(P, bits, ldx_pad=0, ldq_pad=0, ldqT_pad=0):
    t = torch()
    T, C = bits.shape
    xd = bf16_dev(np.pad(bits, ((0, 0), (0, ldx_pad)))) if ldx_pad else bf16_dev(bits)
    qb = t.full((T, C + ldq_pad), 0xA5, dtype=t.uint8, device="cuda")
    qTb = t.full((C, T + ldqT_pad), 0x5A, dtype=t.uint8, device="cuda")
    s = t.full((C // 128, T), float("nan"), dtype=t.float32, device="cuda")
    sT = t.full((T // 128, C), float("nan"), dtype=t.float32, device="cuda")
    P.puro_fp8_quant_act_dual(xd[:, :C], qb[:, :C], s, qTb[:, :T], sT)
    qh, qTh = host(qb), host(qTb)
    assert (qh[:, C:] == 0xA5).all(), "write outside a row of q"
    assert (qTh[:, T:] == 0x5A).all(), "write outside a row of qT"
    return qh[:, :C], host(s), qTh[:, :T], host(sT)


def check_dual(P, bits, what, **kw):
    say(f"[quant dual] {what} shape={bits.shape} {kw}")
    q, s, qT, sT = run_dual(P, bits, **kw)
    rq, rs = quant.quant_act_1x128(bits)
    rqT, rsT = quant.quant_act_128x1(bits)
    assert_bytes_equal(s, rs, f"{what} row scales")
    assert_bytes_equal(q, rq, f"{what} row codes")
    assert_bytes_equal(sT, rsT, f"{what} column scales")
    assert_bytes_equal(qT, rqT, f"{what} transposed codes")


def test_dual_tiny_workload(P):
    check_dual(P, draw("tiny")["X"], "tiny X (outliers)")


@pytest.mark.parametrize("name,tensor", [("qkv_fwd", "X"), ("down_bwd", "dY"), ("down_bwd", "H")])
def test_dual_workloads(P, name, tensor):
    check_dual(P, draw(name)[tensor], f"{name}.{tensor}")


@pytest.mark.parametrize("T,C", [(128, 128), (128, 1280), (384, 256), (1280, 384), (256, 2048)])
def test_dual_shapes(P, T, C):
    rng = np.random.default_rng(T * 7 + C)
    check_dual(P, bf16(rng.standard_t(3, (T, C))), f"student-t {T}x{C}")


def test_dual_strided(P):
    rng = np.random.default_rng(3)
    check_dual(P, bf16(rng.standard_normal((384, 512)) * 1e-3), "strided", ldx_pad=72, ldq_pad=32, ldqT_pad=48)


def test_dual_every_bf16_amax(P):
    # every finite positive bf16 amax appears once as a 1x128 tile amax
    rng = np.random.default_rng(11)
    amax_bits = np.arange(1, 0x7F80, dtype=np.uint16)            # 32639 values
    n = len(amax_bits)
    T = 128 * ((n + 127) // 128)
    base = bf16(rng.uniform(-1, 1, (T, 128)))
    # row r: magnitudes clipped to amax_bits[r], one element set to it exactly
    a = np.concatenate([amax_bits, np.full(T - n, 0x3F80, np.uint16)])
    mag = np.minimum(base & np.uint16(0x7FFF), a[:, None])
    xb = (base & np.uint16(0x8000)) | mag
    pos = rng.integers(0, 128, size=T)
    xb[np.arange(T), pos] = a
    check_dual(P, xb.astype(np.uint16), "every bf16 amax")


def test_dual_zero_denormal_huge_and_outliers(P):
    x = np.zeros((256, 256), np.float32)
    x[1, :] = -0.0
    x[2, :128] = 1e-39
    x[3, :] = 3.3e38
    x[3, 5] = -3.38e38
    x[4, :] = 2.0 ** -96
    x[5, :] = np.linspace(-1e-30, 1e-30, 256)
    x[130:140, 7] = 1e4
    x[200, 200] = -2.5
    x[:, 100] = 1e-39
    check_dual(P, bf16(x), "zero/denormal/huge/outliers")


def test_dual_nonfinite_reading(P):
    x = np.ones((256, 256), np.float32)
    x[3, 10] = np.nan
    x[140, 130] = np.inf
    q, s, qT, sT = run_dual(P, bf16(x))
    assert np.isnan(s[0, 3]) and e4m3.is_nan_code(q[3, :128]).all()
    assert np.isnan(sT[0, 10]) and e4m3.is_nan_code(qT[10, :128]).all()
    assert s[1, 140] == np.inf and sT[1, 130] == np.inf
    assert e4m3.is_nan_code(q[140, 130]) and e4m3.is_nan_code(qT[130, 140])
    rq, rs = quant.quant_act_1x128(bf16(x))
    rqT, rsT = quant.quant_act_128x1(bf16(x))
    assert_bytes_equal(q[200], rq[200], "finite row codes")
    assert_bytes_equal(qT[200], rqT[200], "finite column codes")


def test_dual_matches_single_quantizers(P):
    rng = np.random.default_rng(5)
    bits = bf16(rng.standard_t(3, (512, 768)) * 0.1)
    x = bf16_dev(bits)
    q, s, qT, sT = P.puro_fp8_quant_act_dual(x)
    q1, s1 = P.puro_fp8_quant_act_1x128(x)
    qT1, sT1 = P.puro_fp8_quant_act_128x1(x)
    for a, b, what in ((q, q1, "q"), (s, s1, "s"), (qT, qT1, "qT"), (sT, sT1, "sT")):
        assert_bytes_equal(host(a), host(b), what)


@pytest.mark.parametrize("case", range(12))
def test_dual_random_shape_sweep(P, case):
    """Seeded random shapes (token and column counts in multiples of 128, odd block counts
    included), scales spread over many binades across rows and columns, and padded leading
    dimensions of x, q and qT: all four outputs byte-identical to the oracle."""
    rng = np.random.default_rng(7000 + case)
    T = 128 * int(rng.integers(1, 12))
    C = 128 * int(rng.integers(1, 12))
    x = rng.standard_t(3, size=(T, C)) * np.exp2(rng.integers(-20, 20, size=(T, 1)) + rng.integers(-8, 8, size=(1, C)))
    pads = {"ldx_pad": 8 * int(rng.integers(0, 3)), "ldq_pad": 16 * int(rng.integers(0, 3)),
            "ldqT_pad": 16 * int(rng.integers(0, 3))}
    check_dual(P, bf16(x), f"sweep {case}", **pads)

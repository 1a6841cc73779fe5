"""Pins of the oracle quantizers (CPU only): closed forms, bounds, invariants.

None of these re-types the oracle's formulas: each checks a consequence that the
format and the method fix (exact scaled integers, the half-ulp error bound, a
448 code in every tile, per-tile isolation, transpose invariance), or an exact
rational computation of the IEEE operations.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import e4m3, quant
from workloads import draw, f32_to_bf16_bits

RNG = np.random.default_rng(2024)


def bf16(x):
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def test_bf16_generator_matches_torch_rounding():
    # the shared input generator's float32 -> bf16 rounding against torch's own conversion
    x = RNG.standard_normal(1 << 16).astype(np.float32) * np.float32(3.7)
    x = np.concatenate([x, np.array([0.0, -0.0, 1e-40, -3e38, 65504.0, 1.00390625, 1.01171875], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bf16(x), ref)


def test_bf16_widening_exact():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = quant.bf16_bits_to_f32(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float32).numpy()
    fin = np.isfinite(ref)
    np.testing.assert_array_equal(f[fin], ref[fin])
    assert (np.isnan(f) == np.isnan(ref)).all()


def _exact_f32_round(q: Fraction) -> np.float32:
    """Correctly rounded (RNE) float32 of a positive rational, by exact comparison."""
    c = np.float32(float(q))
    cands = [np.nextafter(c, np.float32(0)), c, np.nextafter(c, np.float32(np.inf))]
    best = None
    for x in cands:
        d = abs(Fraction(float(x)) - q)
        key = (d, int(np.array(x).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, x)
    return best[1]


def test_tile_scale_is_correctly_rounded_for_every_bf16_amax():
    """All 32640 finite non-negative bf16 amax values: s and r are the exact RNE fp32 quotients."""
    bits = np.arange(0x7F80, dtype=np.uint16)            # 0x0000 .. 0x7F7F
    amax = quant.bf16_bits_to_f32(bits)
    s, r = quant.tile_scale(amax)
    floor = Fraction(2) ** -96
    for i in range(len(bits)):
        a = max(Fraction(float(amax[i])), floor)
        assert s[i] == _exact_f32_round(a / 448), (hex(bits[i]), s[i])
        assert r[i] == _exact_f32_round(448 / a), (hex(bits[i]), r[i])
    # all values: s is normal and finite, r*amax rounds back to ~448
    assert np.isfinite(s).all() and (s > 0).all() and np.isfinite(r).all()
    assert (s >= np.float32(2.0 ** -96 / 448 * (1 - 2 ** -23))).all()


@pytest.mark.parametrize("p", [-100, -40, -9, -1, 0, 3, 20, 90])
def test_scaled_small_integers_quantize_exactly(p):
    """Tile = k_i * 2^p with every k_i an E4M3 value and one element = 448 * 2^p.

    Then amax = 448 * 2^p, s = 2^p and r = 2^-p exactly, the scaled values are the
    k_i themselves, and dequantization returns x exactly.
    """
    t = e4m3.decode_table()
    finite = np.array([c for c in range(256) if not np.isnan(t[c])])
    ks = t[RNG.choice(finite, size=(4, 128))]
    ks[:, 5] = 448.0
    x = (ks * 2.0 ** p).astype(np.float32)
    xb = bf16(x)
    assert np.array_equal(quant.bf16_bits_to_f32(xb), x)          # representable in bf16
    q, s = quant.quant_act_1x128(xb)
    assert (s == np.float32(2.0 ** p)).all()
    expect_codes = np.array([[int(np.where((t == k) & (np.signbit(t) == np.signbit(k)))[0][0]) for k in row]
                             for row in ks], dtype=np.uint8)
    np.testing.assert_array_equal(q, expect_codes)
    np.testing.assert_array_equal(e4m3.decode(q) * 2.0 ** p, x.astype(np.float64))


def _ulp_e4m3(a):
    ex = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    return 2.0 ** (ex - 3)


@pytest.mark.parametrize("shape,tile", [((64, 512), (1, 128)), ((256, 96), (128, 1)), ((256, 384), (128, 128))])
def test_error_bound_and_448_code(shape, tile):
    x = (RNG.standard_t(3, size=shape) * 10.0 ** RNG.integers(-8, 8, size=(shape[0], 1))).astype(np.float32)
    xb = bf16(x)
    xf = quant.bf16_bits_to_f32(xb).astype(np.float64)
    q, s = quant.quantize_tiles(xb, *tile)
    s_full = np.repeat(np.repeat(s.astype(np.float64), tile[0], 0), tile[1], 1)
    d = e4m3.decode(q) * s_full
    v = np.abs(xf) / s_full
    bound = s_full * (_ulp_e4m3(v) / 2 + 2.0 ** -21 * v)
    assert (np.abs(xf - d) <= bound).all()
    # every tile whose amax is above the floor contains a +-448 code
    R, C = shape
    qt = q.reshape(R // tile[0], tile[0], C // tile[1], tile[1])
    has448 = ((qt & 0x7F) == 0x7E).any(axis=(1, 3))
    assert has448.all()


def test_zero_and_denormal_tiles():
    x = np.zeros((2, 128), np.float32)
    x[1, :] = -0.0
    x[1, 7] = -1e-40                                      # fp32 denormal, not representable... bf16 keeps it
    xb = bf16(x)
    q, s = quant.quant_act_1x128(xb)
    assert (s == np.float32(2.0 ** -96) / np.float32(448)).all()
    assert (q[0] == 0x00).all() and (q[1] == 0x80).all()


def test_tile_isolation_outlier():
    """One outlier changes only its own tile's scale and codes (per-block scales)."""
    x = RNG.standard_normal((256, 512)).astype(np.float32)
    xb = bf16(x)
    q0, s0 = quant.quant_w_128x128(xb)[:2]
    x2 = x.copy()
    x2[130, 300] = 1e4
    q1, s1 = quant.quant_w_128x128(bf16(x2))[:2]
    changed = s0 != s1
    assert changed.sum() == 1 and changed[1, 2]
    diff = q0 != q1
    assert diff[128:256, 256:384].any()
    diff[128:256, 256:384] = False
    assert not diff.any()
    # same for 1x128 groups
    a0, t0 = quant.quant_act_1x128(xb)
    a1, t1 = quant.quant_act_1x128(bf16(x2))
    assert (t0 != t1).sum() == 1 and t0[2, 130] != t1[2, 130]
    d = a0 != a1
    d[130, 256:384] = False
    assert not d.any()


def test_blockwise_error_below_per_tensor_error_on_outlier_workload():
    """Reported statistic: 128x128 / 1x128 scales beat one per-tensor scale on the outlier input."""
    X = draw("tiny")["X"]
    xf = quant.bf16_bits_to_f32(X).astype(np.float64)
    q, s = quant.quant_act_1x128(X)
    blk = e4m3.decode(q) * np.repeat(s.T.astype(np.float64), 128, axis=1)
    qt, st = quant.quantize_tiles(X, X.shape[0], X.shape[1])        # one tile = per-tensor scale
    ten = e4m3.decode(qt) * float(st[0, 0])
    assert np.abs(blk - xf).mean() < np.abs(ten - xf).mean()


def test_transpose_invariants():
    x = bf16(RNG.standard_normal((384, 256)).astype(np.float32) * 3)
    # 128x1 on X equals 1x128 on X^T (bytes and scales)
    qT, sT = quant.quant_act_128x1(x)
    q2, s2 = quant.quant_act_1x128(np.ascontiguousarray(x.T))
    np.testing.assert_array_equal(qT, q2)
    np.testing.assert_array_equal(sT, s2)
    # weight blocks: quantizing W^T gives the transposed codes and scales
    q, s, wqT, wsT = quant.quant_w_128x128(x)
    q3, s3 = quant.quantize_tiles(np.ascontiguousarray(x.T), 128, 128)
    np.testing.assert_array_equal(wqT, q3)
    np.testing.assert_array_equal(wsT, s3)
    np.testing.assert_array_equal(wqT, q.T)
    # block scale is the max of the 1x128 scales of its rows (fl32 division is monotone)
    _, sg = quant.quant_act_1x128(x)                   # [K/128, M]
    blockmax = sg.T.reshape(3, 128, 2).max(axis=1)     # [M/128, K/128]
    np.testing.assert_array_equal(s, blockmax)


def test_nonfinite_reading():
    x = np.ones((3, 128), np.float32)
    x[0, 3] = np.nan
    x[1, 4] = np.inf
    x[2, 5] = -np.inf
    q, s = quant.quant_act_1x128(bf16(x))
    assert np.isnan(s[0, 0]) and e4m3.is_nan_code(q[0]).all()
    assert s[0, 1] == np.inf and s[0, 2] == np.inf
    assert e4m3.is_nan_code(q[1, 4]) and e4m3.is_nan_code(q[2, 5])
    assert (q[1, [0, 1, 2, 3, 5]] == 0x00).all()

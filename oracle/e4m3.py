"""OCP FP8 E4M3 ("e4m3fn") decode table and two independent fp32 -> E4M3 encoders.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this module.

Format (public OCP 8-bit Floating Point Specification, OFP8, E4M3 variant; the
pages only say "FP8", see the readings list in the design notes):
  bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0 mantissa;
  exponent 0       -> subnormal  (m/8) * 2^-6
  exponent 1..15   -> normal     (1 + m/8) * 2^(e-7)
  S.1111.111       -> NaN (the only NaN pattern per sign; there is no infinity)
  largest finite magnitude 448 = S.1111.110.

The quantizer's cast is "round to nearest, ties to even, saturating": the
nearest representable magnitude is taken, a tie goes to the code whose least
significant bit is 0, magnitudes at or above 448 give 448, the sign bit is
kept (also when the magnitude rounds to zero), NaN gives a NaN code.

``encode_nearest`` follows that definition literally (search the 127
non-negative finite magnitudes, compare against the midpoints).
``encode_bits`` reaches the same result by integer arithmetic on the fp32 bit
fields.  They share nothing but the decode table's constants, and the tests pin
them against each other, against the table, and against PyTorch's own
``float8_e4m3fn`` conversion.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
CODE_MAX = 0x7E   # +448
CODE_NAN = 0x7F   # +NaN (sign bit may also be set)


def decode_table() -> np.ndarray:
    """float64 value of each of the 256 codes, built from the bit fields."""
    out = np.empty(256, dtype=np.float64)
    for c in range(256):
        s = (c >> 7) & 1
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            v = np.nan
        elif e == 0:
            v = (m / 8.0) * 2.0 ** -6
        else:
            v = (1.0 + m / 8.0) * 2.0 ** (e - 7)
        out[c] = -v if s else v
    return out


_TABLE = decode_table()
_MAGS = _TABLE[: CODE_MAX + 1].copy()           # codes 0x00..0x7E, strictly increasing
_MIDS = 0.5 * (_MAGS[:-1] + _MAGS[1:])          # exact in float64 (<= 5 significant bits)


def decode(codes: np.ndarray) -> np.ndarray:
    """float64 values of uint8 codes."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def encode_nearest(v: np.ndarray) -> np.ndarray:
    """Saturating round-to-nearest-even encode by searching the magnitude table.

    ``v`` is float32 (any shape).  The magnitude is compared, exactly, against
    the midpoints between consecutive representable magnitudes.
    """
    v = np.asarray(v, dtype=np.float32)
    with np.errstate(invalid="ignore"):
        a = np.abs(v.astype(np.float64))
    nan = np.isnan(a)
    a_safe = np.where(nan, 0.0, a)
    # hi = index of the first magnitude >= a  (clamped into [1, 126]); lo = hi - 1
    hi = np.searchsorted(_MAGS, a_safe, side="left")
    hi = np.clip(hi, 1, CODE_MAX)
    lo = hi - 1
    mid = _MIDS[lo]
    pick_hi = a_safe > mid
    tie = a_safe == mid
    pick_hi = pick_hi | (tie & ((lo & 1) == 1))      # tie -> the even code
    code = np.where(pick_hi, hi, lo).astype(np.int64)
    code = np.where(a_safe >= E4M3_MAX, CODE_MAX, code)  # saturate (also +-inf)
    code = np.where(nan, CODE_NAN, code)
    sign = np.signbit(v).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)


def encode_bits(v: np.ndarray) -> np.ndarray:
    """Saturating round-to-nearest-even encode by integer arithmetic on the fp32 bits.

    Normal E4M3 range: keep the implicit one plus 3 mantissa bits, i.e. drop the
    low 20 bits of the 24-bit significand with RNE.  Below 2^-6 the grid is the
    subnormal step 2^-9: the significand is shifted right by 14 - unbiased_exp.
    """
    v = np.asarray(v, dtype=np.float32)
    u = v.view(np.uint32).astype(np.int64)
    sign = (u >> 31) & 1
    e = (u >> 23) & 0xFF
    m = u & 0x7FFFFF
    ue = e - 127
    sig = m | (1 << 23)

    # normal target (ue >= -6)
    q_n = sig >> 20
    rem_n = sig & ((1 << 20) - 1)
    up_n = (rem_n > (1 << 19)) | ((rem_n == (1 << 19)) & ((q_n & 1) == 1))
    q_n = q_n + up_n
    carry = q_n == 16
    q_n = np.where(carry, 8, q_n)
    E = ue + 7 + carry
    code_n = (E << 3) | (q_n & 7)
    over = (E > 15) | ((E == 15) & (q_n > 14))
    code_n = np.where(over, CODE_MAX, code_n)

    # subnormal target (ue < -6): value in units of 2^-9 is sig * 2^(ue - 14)
    shift = np.clip(14 - ue, 1, 40)
    q_s = sig >> np.minimum(shift, 63)
    rem_s = sig & ((np.int64(1) << shift) - 1)
    half = np.int64(1) << (shift - 1)
    up_s = (rem_s > half) | ((rem_s == half) & ((q_s & 1) == 1))
    code_s = q_s + up_s               # q_s + up in 0..8; 8 is the smallest normal 0x08

    code = np.where(ue >= -6, code_n, code_s)
    code = np.where(e == 0, 0, code)                     # fp32 zero / subnormal -> 0
    code = np.where((e == 0xFF) & (m == 0), CODE_MAX, code)  # +-inf saturates
    code = np.where((e == 0xFF) & (m != 0), CODE_NAN, code)  # NaN
    return (code | (sign << 7)).astype(np.uint8)


def is_nan_code(c: np.ndarray) -> np.ndarray:
    return (np.asarray(c, dtype=np.uint8) & 0x7F) == 0x7F

"""Exact decoders/encoder for the stored number formats (test infrastructure).

bf16 and fp8 are the cache formats the path reads.  The pages name "cache
precision" as a variable to control ([ES-lim]) and the deployment they report
runs FP8; which fp8 variant is not stated.  Reading taken: OCP E4M3FN
(1 sign, 4 exponent bits with bias 7, 3 mantissa bits, subnormals, no
infinities, the all-ones pattern S.1111.111 is NaN, largest finite 448),
with a per-tensor fp32 scale: value = decode(code) * scale.  The same
per-tensor scale form is kept for a bf16 cache (scale 1 unless stated).
"""

import numpy as np

FP8_MAX = 448.0


def bf16_to_f64(u16):
    """bf16 bit patterns (uint16) -> exact float64 values.

    A bf16 number is the top half of an IEEE binary32 number, so the exact
    value is the binary32 number whose low 16 bits are zero.
    """
    u16 = np.asarray(u16, dtype=np.uint16)
    u32 = u16.astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def _fp8_decode_scalar(c):
    """Value of one E4M3FN code, straight from the bit fields."""
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        mag = (m / 8.0) * 2.0 ** (1 - 7)          # subnormal: 0.m * 2^(1-bias)
    else:
        mag = (1.0 + m / 8.0) * 2.0 ** (e - 7)    # normal: 1.m * 2^(e-bias)
    return -mag if s else mag


_FP8_TABLE = np.array([_fp8_decode_scalar(c) for c in range(256)], dtype=np.float64)
# Non-negative finite codes 0x00..0x7E in increasing value order.
_FP8_POS = _FP8_TABLE[:0x7F].copy()


def fp8_decode(codes):
    """E4M3FN codes (uint8) -> exact float64 values (NaN for 0x7F/0xFF)."""
    codes = np.asarray(codes, dtype=np.uint8)
    return _FP8_TABLE[codes]


def fp8_encode(x):
    """float64 -> E4M3FN codes: round to nearest, ties to the even code,
    saturating at +-448; NaN -> 0x7F.

    Written as a nearest-neighbour search over the 127 non-negative finite
    grid values.  Adjacent codes differ by one in the integer code, so "ties
    to even" means ties go to the even code (whose last mantissa bit is 0).
    The sign is kept, so values that round to zero give +0 or -0 (0x80).
    """
    x = np.asarray(x, dtype=np.float64)
    mag = np.abs(x)
    sign = np.signbit(x)
    # index of the first grid value >= mag (clipped to the grid)
    hi = np.searchsorted(_FP8_POS, np.minimum(mag, FP8_MAX), side="left")
    hi = np.clip(hi, 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    d_lo = np.abs(mag - _FP8_POS[lo])
    d_hi = np.abs(_FP8_POS[hi] - mag)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.int64)
    code = np.where(mag >= FP8_MAX, 0x7E, code)
    code = np.where(sign, code | 0x80, code)
    code = np.where(np.isnan(x), 0x7F, code)
    return code.astype(np.uint8)

"""Pins for the oracle's number-format codecs (CPU only).

The fp8 cache format is a reading (OCP E4M3FN; the pages only say the
deployment runs FP8 and that cache precision matters).  These tests pin the
oracle's codec to the format's fixed points and to torch's independent
float8_e4m3fn / bfloat16 conversions (library routines).
"""

import numpy as np
import pytest
import torch

from oracle.codec import bf16_to_f64, fp8_decode, fp8_encode, FP8_MAX
from oracle.prologue import bf16_encode


ALL = np.arange(256, dtype=np.uint8)
FINITE = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)


def test_fp8_decode_fixed_points():
    v = fp8_decode(ALL)
    assert v[0x00] == 0.0 and v[0x80] == 0.0 and np.signbit(v[0x80])
    assert v[0x01] == 2.0 ** -9            # smallest subnormal
    assert v[0x07] == 7 * 2.0 ** -9        # largest subnormal
    assert v[0x08] == 2.0 ** -6            # smallest normal
    assert v[0x38] == 1.0                  # exponent field 7 = bias
    assert v[0x7E] == FP8_MAX == 448.0
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)        # strictly monotone
    assert np.array_equal(v[0x80:0xFF], -pos)


def test_fp8_decode_matches_torch():
    t = torch.from_numpy(ALL.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    v = fp8_decode(ALL)
    assert np.array_equal(np.isnan(t), np.isnan(v))
    ok = ~np.isnan(v)
    assert np.array_equal(t[ok], v[ok])


def test_fp8_encode_roundtrip_and_ties():
    assert np.array_equal(fp8_encode(fp8_decode(FINITE)), FINITE)
    pos = fp8_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2
    lo = np.arange(0x7E)
    got = fp8_encode(mids).astype(np.int64)
    want = np.where(lo % 2 == 0, lo, lo + 1)        # ties go to the even code
    assert np.array_equal(got, want)
    eps = 1e-12
    assert np.array_equal(fp8_encode(mids * (1 + eps)).astype(np.int64), lo + 1)
    assert np.array_equal(fp8_encode(mids * (1 - eps)).astype(np.int64), lo)


def test_fp8_encode_saturation_nan_sign():
    assert fp8_encode(np.array([448.0, 449.0, 464.0, 1e30]))[...].tolist() == [0x7E] * 4
    assert fp8_encode(np.array([-448.0, -1e30])).tolist() == [0xFE, 0xFE]
    assert fp8_encode(np.array([np.nan])).tolist() == [0x7F]
    assert fp8_encode(np.array([0.0, -0.0, 2.0 ** -12, -(2.0 ** -12)])).tolist() == [0, 0x80, 0, 0x80]


def test_fp8_encode_matches_torch_on_float32():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 0.05, 1, 30, 200)])
    x = np.clip(x, -448, 448).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(fp8_encode(x.astype(np.float64)), ref)


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 2 ** 16, size=50000, dtype=np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]               # finite patterns only
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(bf16_to_f64(bits), t)


def test_bf16_encode_matches_torch_and_avoids_double_rounding():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(50000) * 3).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16_encode(x.astype(np.float64)), ref)
    # 1 + 2^-8 is the midpoint between bf16 1.0 and 1 + 2^-7.  A value just
    # above it must round up; a detour through float32 would land exactly on
    # the midpoint and round down to even.
    assert bf16_encode(np.array([1 + 2.0 ** -8 + 2.0 ** -30])).tolist() == [0x3F81]
    assert bf16_encode(np.array([1 + 2.0 ** -8])).tolist() == [0x3F80]
    assert bf16_encode(np.array([1 + 3 * 2.0 ** -8])).tolist() == [0x3F82]

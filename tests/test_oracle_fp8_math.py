"""Pins for the native-fp8 oracle (CPU only).

q quantisation is checked against the format (the largest element maps to
448, every code is the nearest-even grid point, the scale is amax / 448 in
float32) and is the identity on values already on the scaled fp8 grid.  The
weight-rounding bound is checked against a simulation of the rounding the
method performs (weights of 64-token chunks kept as an E4M3 value plus an
E4M3 residual against the running maximum, online rescaling, normalisation
by the rounded weights),
for flat and sharply peaked score distributions; an understated bound is
planted and must fail.
"""

import numpy as np
import pytest

import oracle
import oracle.fp8_math as fm
from oracle.codec import fp8_decode, fp8_encode
from load_balanced_split_step_amd.workloads import Workload, make_inputs


def test_quantize_q_format():
    rng = np.random.default_rng(0)
    q = (rng.standard_normal((5, 7, 128)) * rng.uniform(0.01, 30, size=(5, 7, 1))).astype(np.float32)
    codes, s_q = fm.quantize_q_fp8(q)
    assert s_q.dtype == np.float32
    assert np.array_equal(s_q, np.abs(q).max(axis=-1) / np.float32(448.0))
    x = (q / s_q[..., None]).astype(np.float32).astype(np.float64)
    i = np.abs(q).reshape(35, 128).argmax(axis=1)
    top = codes.reshape(35, 128)[np.arange(35), i]
    assert np.all((top & 0x7F) == 0x7E)                       # +-448
    dec = fp8_decode(codes)
    # nearest grid point: no code is farther from x than the one next to it
    up = fp8_decode(np.where(codes & 0x7F < 0x7E, codes + 1, codes).astype(np.uint8))
    dn = fp8_decode(np.where(codes & 0x7F > 0, codes - 1, codes).astype(np.uint8))
    assert np.all(np.abs(dec - x) <= np.abs(up - x) + 0.0)
    assert np.all(np.abs(dec - x) <= np.abs(dn - x) + 0.0)
    normal = np.abs(x) >= 2.0 ** -6
    assert np.all(np.abs(dec - x)[normal] <= 2.0 ** -4 * np.abs(x)[normal])


def test_quantize_q_residual_format():
    """The residual codes are the nearest-even E4M3 grid points of
    16 (x - decode(hi)); the split hi + lo/16 lies within 2^-8 |x| + 2^-14 of
    x (E4M3's relative rounding 2^-4 taken twice, plus the residual's
    subnormal floor 2^-10 / 16), eight times closer than hi alone; planted
    mistakes in the residual's scale (dropped, applied twice) break the
    bound."""
    rng = np.random.default_rng(3)
    q = (rng.standard_normal((6, 5, 128)) * rng.uniform(1e-3, 50, size=(6, 5, 1))).astype(np.float32)
    q[0, 0, :7] = [0.0, 1e-9, -3e-7, 2.0 ** -20, 5e-5, -1e-4, 3e-3]   # subnormal residuals
    hi, s_q = fm.quantize_q_fp8(q)
    lo = fm.quantize_q_residual(q)
    x = np.clip((q / s_q[..., None]).astype(np.float32), -448, 448).astype(np.float64)
    r16 = 16.0 * (x - fp8_decode(hi))
    assert np.abs(r16).max() <= 256.0                        # inside E4M3's range
    dec = fp8_decode(lo)
    up = fp8_decode(np.where(lo & 0x7F < 0x7E, lo + 1, lo).astype(np.uint8))
    dn = fp8_decode(np.where(lo & 0x7F > 0, lo - 1, lo).astype(np.uint8))
    assert np.all(np.abs(dec - r16) <= np.abs(up - r16)) and np.all(np.abs(dec - r16) <= np.abs(dn - r16))
    bound = 2.0 ** -8 * np.abs(x) + 2.0 ** -14
    eff = fp8_decode(hi) + dec / 16.0
    assert np.all(np.abs(eff - x) <= bound)
    assert np.abs(eff - x).max() <= np.abs(fp8_decode(hi) - x).max() / 8
    for bad in (fp8_decode(hi) + dec, fp8_decode(hi) + dec / 256.0):      # planted
        assert not np.all(np.abs(bad - x) <= bound)
    np.testing.assert_array_equal(fm.dequantized_q(q), eff * s_q.astype(np.float64)[..., None])


def test_quantize_q_zero_row():
    q = np.zeros((1, 2, 64), np.float32)
    q[0, 1, 3] = -2.5
    codes, s_q = fm.quantize_q_fp8(q)
    assert s_q[0, 0] == 1.0 and not codes[0, 0].any()
    assert codes[0, 1, 3] == 0xFE and s_q[0, 1] == np.float32(2.5) / np.float32(448)
    assert not fm.quantize_q_residual(q).any()


def test_quantization_is_identity_on_the_grid():
    """q = 2^-3 * decode(c) with a +-448 code in every row: s_q = 2^-3
    exactly, so the codes come back unchanged and attention_fp8q equals the
    exact attention with q itself."""
    w = Workload("q8", 3, 8, 2, 16, 16, kv_dtype="fp8", seed=50)
    inp = make_inputs(w, lengths=[20, 33, 7])
    rng = np.random.default_rng(1)
    c = rng.integers(0, 0x7F, size=(3, 8, 16)).astype(np.uint8)
    c[..., 5] = 0x7E
    c |= (rng.integers(0, 2, size=c.shape) * 0x80).astype(np.uint8)
    q = (fp8_decode(c) * 2.0 ** -3).astype(np.float32)
    codes, s_q = fm.quantize_q_fp8(q)
    assert np.all(s_q == np.float32(0.125)) and np.array_equal(codes, c)
    assert not fm.quantize_q_residual(q).any()               # nothing left for the residual
    args = (inp["k_pages"], inp["v_pages"], inp["block_table"], inp["seq_lens"], "fp8",
            float(inp["sm_scale"]))
    kw = dict(k_scale=float(inp["k_scale"]), v_scale=float(inp["v_scale"]))
    np.testing.assert_allclose(fm.attention_fp8q(q, *args, **kw),
                               oracle.attention_reference(q.astype(np.float64), *args, **kw),
                               rtol=0, atol=1e-12)


def _simulate(s, v, chunk=64):
    """Online softmax over chunks with each chunk's weights z = p * 2^8,
    against the running maximum, kept as E4M3(z) plus E4M3 of the residual;
    returns o'."""
    m = -np.inf
    acc = np.zeros(v.shape[1])
    l = 0.0
    for c0 in range(0, len(s), chunk):
        sc = s[c0:c0 + chunk]
        m_new = max(m, sc.max())
        alpha = np.exp(m - m_new) if np.isfinite(m) else 0.0
        z = np.exp(sc - m_new) * 256.0
        a = fp8_decode(fp8_encode(z))
        p8 = (a + fp8_decode(fp8_encode(z - a))) / 256.0
        acc = acc * alpha + p8 @ v[c0:c0 + chunk]
        l = l * alpha + p8.sum()
        m = m_new
    return acc / l


def _cases():
    rng = np.random.default_rng(2)
    for L, sharp in [(5, 1.0), (64, 1.0), (300, 3.0), (2000, 1.0), (3000, 8.0), (5000, 20.0)]:
        s = rng.standard_normal(L) * sharp
        if sharp > 5:                      # a few dominant keys, most weights below 2^-14
            s[rng.integers(0, L, 3)] += 40.0
        v = rng.standard_normal((L, 32))
        yield s, v


def _bound(s, v, u):
    p = np.exp(s - s.max())
    z = p.sum()
    o = (p @ v) / z
    dev = np.abs(v - o)
    worst = (u * (p @ dev) + fm.SUB_ABS * dev.sum(axis=0)) / ((1 - u) * z)
    w = p / z
    rms = np.sqrt((u * u / 3) * ((w * w) @ (dev * dev)))
    return o, worst, rms


def test_bound_holds_under_simulated_rounding():
    err2, pred2 = 0.0, 0.0
    for s, v in _cases():
        o, worst, rms = _bound(s, v, fm.U_WEIGHTS)
        e = np.abs(_simulate(s, v) - o)
        assert np.all(e <= worst + 1e-15), float((e / worst).max())
        err2 += float((e * e).sum())
        pred2 += float((rms * rms).sum())
    assert err2 <= 4.0 * pred2, (err2, pred2)


def test_bound_matches_oracle_function():
    """weight_rounding_bounds computes the same bound from a paged cache."""
    w = Workload("bnd", 2, 4, 2, 16, 16, kv_dtype="fp8", seed=51)
    inp = make_inputs(w, lengths=[70, 300])
    q = fm.dequantized_q(inp["q"])
    pairs = [(0, 0), (1, 3)]
    res = fm.weight_rounding_bounds(q, inp["k_pages"], inp["v_pages"], inp["block_table"],
                                    inp["seq_lens"], "fp8", float(inp["sm_scale"]), pairs,
                                    float(inp["k_scale"]), float(inp["v_scale"]))
    ref = oracle.attention_selected(q, inp["k_pages"], inp["v_pages"], inp["block_table"],
                                    inp["seq_lens"], "fp8", float(inp["sm_scale"]), pairs,
                                    float(inp["k_scale"]), float(inp["v_scale"]))
    for key in pairs:
        o, worst, rms = res[key]
        np.testing.assert_allclose(o, ref[key], rtol=0, atol=1e-12)
        assert np.all(worst > 0) and np.all(rms > 0) and np.all(rms <= worst)


def test_weight_split_error():
    """z = p 2^8 kept as a = E4M3(z) plus b = E4M3(z - a): within 2^-8 z +
    2^-10 of z over [0, 256] (sixteen times tighter than a alone in the
    normal range); dropping the residual breaks that bound."""
    z = np.concatenate([np.linspace(0, 256, 200001), np.exp(np.linspace(-30, np.log(256), 5001))])
    a = fp8_decode(fp8_encode(z))
    ab = a + fp8_decode(fp8_encode(z - a))
    assert np.all(np.abs(ab - z) <= 2.0 ** -8 * z + 2.0 ** -10)
    assert not np.all(np.abs(a - z) <= 2.0 ** -8 * z + 2.0 ** -10)         # planted: no residual
    normal = z >= 2.0 ** -6
    assert np.abs(ab - z)[normal].max() * 16 <= np.abs(a - z)[normal].max()


def test_planted_understated_bound_is_caught():
    caught = False
    for s, v in _cases():
        o, worst, _ = _bound(s, v, 2.0 ** -11)
        if np.any(np.abs(_simulate(s, v) - o) > worst):
            caught = True
    assert caught

"""Pins for the oracle's RMSNorm, RoPE and new-token prologue (CPU only).

Pinned against torch's rms_norm (a library routine), closed forms of the
rotation (identity at position 0, norm preservation, the relative-position
identity), hand-worked rotation values for a 4-dim head, and the cache-write
layout.
"""

import math

import numpy as np
import pytest
import torch

from oracle.codec import bf16_to_f64, fp8_decode, fp8_encode
from oracle.prologue import rms_norm, rope, prologue_step, write_new_token, bf16_encode
from load_balanced_split_step_amd.workloads import Workload, make_inputs


def test_rms_norm_matches_torch():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 7, 128))
    w = rng.normal(1, 0.1, 128)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (128,), torch.from_numpy(w), eps=1e-6).numpy()
    np.testing.assert_allclose(rms_norm(x, w, 1e-6), ref, rtol=1e-14, atol=1e-14)


def test_rms_norm_unit_weight_closed_form():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((9, 64)) * 0.01
    eps = 1e-6
    y = rms_norm(x, np.ones(64), eps)
    ms = np.mean(x * x, axis=-1)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), (1 + eps / ms) ** -0.5, rtol=1e-13)


def test_rope_position_zero_is_identity():
    x = np.random.default_rng(3).standard_normal((4, 128))
    assert np.array_equal(rope(x, np.zeros(4), 1e6), x)


def test_rope_preserves_norm_and_relative_position():
    rng = np.random.default_rng(4)
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    for style in ("rotate_half", "interleaved"):
        for m, n in [(5, 2), (32767, 100), (1000, 999)]:
            qm = rope(q, np.array(m), 1e6, style)
            kn = rope(k, np.array(n), 1e6, style)
            np.testing.assert_allclose(np.linalg.norm(qm), np.linalg.norm(q), rtol=1e-13)
            rel = rope(q, np.array(m - n), 1e6, style)
            np.testing.assert_allclose(qm @ kn, rel @ k, rtol=1e-9, atol=1e-9)


def test_rope_hand_worked_d4():
    # D = 4, theta = 1e6: frequencies theta^0 = 1 and theta^(-1/2) = 1e-3.
    # Rotate-half pairs dims (0, 2) by pos*1 and (1, 3) by pos*1e-3.
    e = np.eye(4)
    y0 = rope(e[0], np.array(1.0), 1e6)
    np.testing.assert_allclose(y0, [0.5403023058681398, 0, 0.8414709848078965, 0], atol=1e-15)
    y1 = rope(e[1], np.array(1.0), 1e6)
    np.testing.assert_allclose(y1, [0, 0.9999995000000417, 0, 0.0009999998333333417], atol=1e-15)
    y2 = rope(e[2], np.array(2.0), 1e6)   # (x0, x2) = (0, 1) rotated by 2 rad
    np.testing.assert_allclose(y2, [-0.9092974268256817, 0, -0.4161468365471424, 0], atol=1e-15)
    # the interleaved form pairs (0, 1) instead and gives a different vector
    assert not np.allclose(rope(e[0], np.array(1.0), 1e6, "interleaved"), y0)


def _prologue_inputs(kv):
    w = Workload("pro", 5, 8, 2, 128, 16, kv_dtype=kv, prologue=True, seed=40)
    return make_inputs(w, lengths=[1, 16, 17, 300, 64])


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_prologue_codes_round_the_normed_rotated_values(kv):
    inp = _prologue_inputs(kv)
    q_p, k_p, v, kc, vc = prologue_step(inp["q"], inp["k_new"], inp["v_new"], inp["q_norm_w"],
                                        inp["k_norm_w"], inp["seq_lens"], float(inp["rms_eps"]),
                                        float(inp["rope_theta"]), kv, float(inp["k_scale"]),
                                        float(inp["v_scale"]))
    # k' is RoPE(RMSNorm(k)) at pos = len - 1
    pos = inp["seq_lens"].astype(np.int64) - 1
    kf = bf16_to_f64(inp["k_new"])
    wk = bf16_to_f64(inp["k_norm_w"])
    y = kf / np.sqrt(np.mean(kf ** 2, axis=-1, keepdims=True) + 1e-6) * wk
    np.testing.assert_allclose(k_p, rope(y, pos[:, None], 1e6), rtol=1e-12, atol=1e-12)
    # norm per head after RoPE equals norm before (rotation)
    np.testing.assert_allclose(np.linalg.norm(k_p, axis=-1), np.linalg.norm(y, axis=-1), rtol=1e-12)
    if kv == "fp8":
        ks, vs = float(inp["k_scale"]), float(inp["v_scale"])
        # the stored code is the nearest grid point: error within half a step
        for codes, x, s in [(kc, k_p / ks, ks), (vc, v / vs, vs)]:
            dec = fp8_decode(codes)
            err = np.abs(dec - np.clip(x, -448, 448))
            grid = fp8_decode(np.arange(127, dtype=np.uint8))
            gaps = np.diff(grid)
            j = np.searchsorted(grid, np.abs(dec))
            step = np.maximum(gaps[np.clip(j - 1, 0, 125)], gaps[np.clip(j, 0, 125)])
            assert np.all(err <= step / 2 + 1e-12)
            # and no other code is closer
            assert np.all(np.abs(fp8_decode(fp8_encode(x)) - np.clip(x, -448, 448)) <= err + 1e-12)
    else:
        np.testing.assert_allclose(bf16_to_f64(kc), k_p, rtol=2 ** -8)


def test_write_new_token_places_slot():
    inp = _prologue_inputs("fp8")
    B, Hkv, D = inp["k_new"].shape
    kc = np.arange(B * Hkv * D, dtype=np.int64).reshape(B, Hkv, D) % 251
    vc = (kc + 3) % 251
    kp, vp = write_new_token(inp["k_pages"], inp["v_pages"], inp["block_table"], inp["seq_lens"],
                             kc.astype(np.uint8), vc.astype(np.uint8))
    ps = kp.shape[2]
    for b, L in enumerate(inp["seq_lens"].tolist()):
        page = inp["block_table"][b][(L - 1) // ps]
        assert np.array_equal(kp[page, :, (L - 1) % ps, :], kc[b])
        assert np.array_equal(vp[page, :, (L - 1) % ps, :], vc[b])
    # nothing else changed
    changed = (kp != inp["k_pages"]).any(axis=(1, 3)).sum()
    assert changed == B

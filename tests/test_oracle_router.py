"""Pins for the Router GEMM oracle (CPU only).

The split against the formats: hi is torch's round-to-nearest-even bf16 cast
of w, lo the same cast of the residual times 256, and hi + lo/256 recovers w
to about 2^-17 relative (16 significant bits); weights already on the bf16
grid split exactly (lo = 0).  The products against a pure-Python brute force
(math.fsum) and closed forms (one-hot activations select weight columns).
The accumulation bound against a float32 evaluation in the worst summation
order for it (sorted by magnitude, large first).  Planted mistakes (residual
scale applied twice, lo dropped) are caught.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import oracle.router as orr
from load_balanced_split_step_amd.workloads import ROUTER_CONFIGS, make_router_inputs


def test_split_against_torch_casts():
    inp = make_router_inputs(ROUTER_CONFIGS["router_small"])
    w = inp["w"]
    hi, lo = orr.split_router_weights(w)
    t_hi = torch.from_numpy(w).to(torch.bfloat16)
    assert np.array_equal(hi, t_hi.view(torch.int16).numpy().view(np.uint16))
    res = (torch.from_numpy(w) - t_hi.to(torch.float32)) * 256.0       # exact in float32
    assert np.array_equal(lo, res.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


def test_split_recovers_weights():
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((40, 300)) * 10.0 ** rng.uniform(-4, 2, (40, 1))).astype(np.float32)
    hi, lo = orr.split_router_weights(w)
    rel = np.abs(orr.split_value(hi, lo) - w.astype(np.float64)) / np.abs(w.astype(np.float64))
    assert rel.max() <= 2.0 ** -16
    on_grid = oracle.bf16_to_f64(hi).astype(np.float32)
    hi2, lo2 = orr.split_router_weights(on_grid)
    assert np.array_equal(hi2, hi) and not lo2.any()


def test_products_against_brute_force():
    inp = make_router_inputs(ROUTER_CONFIGS["router_small"])
    x, w = inp["x"], inp["w"]
    hi, lo = orr.split_router_weights(w)
    xf = oracle.bf16_to_f64(x).tolist()
    wf = w.astype(np.float64).tolist()
    sv = orr.split_value(hi, lo).tolist()
    T, E, H = x.shape[0], w.shape[0], w.shape[1]
    exact = np.array([[math.fsum(xf[t][h] * wf[e][h] for h in range(H)) for e in range(E)]
                      for t in range(T)])
    split = np.array([[math.fsum(xf[t][h] * sv[e][h] for h in range(H)) for e in range(E)]
                      for t in range(T)])
    np.testing.assert_allclose(orr.router_reference(x, w), exact, rtol=0, atol=1e-13)
    np.testing.assert_allclose(orr.router_split_reference(x, hi, lo), split, rtol=0, atol=1e-13)


def test_one_hot_activations_select_columns():
    inp = make_router_inputs(ROUTER_CONFIGS["router_small"])
    w = inp["w"]
    H = w.shape[1]
    x = np.zeros((H, H), np.float32)
    np.fill_diagonal(x, 1.0)
    xb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(orr.router_reference(xb, w), w.T.astype(np.float64))
    hi, lo = orr.split_router_weights(w)
    np.testing.assert_array_equal(orr.router_split_reference(xb, hi, lo), orr.split_value(hi, lo).T)


def test_accumulation_bound_holds_for_float32():
    inp = make_router_inputs(ROUTER_CONFIGS["router"], tokens=3)
    x, w = inp["x"], inp["w"][:8]
    hi, lo = orr.split_router_weights(w)
    ref = orr.router_split_reference(x, hi, lo)
    bound = orr.accumulation_bound(x, hi, lo)
    xf = oracle.bf16_to_f64(x).astype(np.float32)
    for t in range(3):
        for e in range(8):
            out = np.float32(0.0)
            for part, s in ((oracle.bf16_to_f64(hi[e]), 1.0), (oracle.bf16_to_f64(lo[e]), 1 / 256)):
                terms = (xf[t] * part.astype(np.float32)).astype(np.float32)
                acc = np.float32(0.0)
                for v in terms[np.argsort(-np.abs(terms))]:
                    acc = np.float32(acc + v)
                out = np.float32(out + np.float32(acc * np.float32(s)))
            assert abs(float(out) - ref[t, e]) <= bound[t, e]


def test_planted_mistakes_are_caught():
    inp = make_router_inputs(ROUTER_CONFIGS["router_small"])
    x, w = inp["x"], inp["w"]
    hi, lo = orr.split_router_weights(w)
    exact = orr.router_reference(x, w)
    good = orr.router_split_reference(x, hi, lo)
    drop = oracle.bf16_to_f64(x) @ oracle.bf16_to_f64(hi).T                     # lo dropped
    twice = oracle.bf16_to_f64(x) @ (oracle.bf16_to_f64(hi) + oracle.bf16_to_f64(lo) / 65536).T
    err = lambda a: float(np.abs(a - exact).max())
    assert err(good) < 1e-4 * float(np.abs(exact).max())
    assert err(drop) > 20 * err(good) and err(twice) > 20 * err(good)

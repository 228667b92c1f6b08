"""Pins for the oracle attention and its split/merge form (CPU only).

Each pin checks the oracle against something other than itself: a pure-Python
brute force with its own page lookups, closed forms (one token, constant V,
zero query, one dominant key, a score shift), torch's scaled-dot-product
attention (a library routine), page-permutation invariance, and the split
then merge = unsplit identity.  The last tests plant plausible mistakes in
the oracle and check that a pin catches each one.
"""

import math

import numpy as np
import pytest
import torch

import oracle.attention as oa
from oracle import (attention_reference, attention_bruteforce, attention_selected,
                    split_merge_reference, plan_dynamic, plan_static, decode_kv,
                    gather_request)
from load_balanced_split_step_amd.workloads import Workload, make_inputs, CONFIGS


def run_ref(inp, q=None, fn=attention_reference, **kw):
    q64 = oa.bf16_to_f64(inp["q"]) if q is None else q
    return fn(q64, inp["k_pages"], inp["v_pages"], inp["block_table"], inp["seq_lens"],
              inp["kv_dtype"], float(inp["sm_scale"]), k_scale=float(inp["k_scale"]),
              v_scale=float(inp["v_scale"]), scale_mode=inp["scale_mode"],
              k_scales=inp["k_scales"], v_scales=inp["v_scales"], **kw)


SMALL = [
    (CONFIGS["tiny"], None),
    (Workload("mha", 3, 4, 4, 16, 16, seed=11), [1, 33, 50]),
    (Workload("gqa8", 2, 16, 2, 8, 16, seed=12), [40, 17]),
    (Workload("fp8s", 3, 6, 2, 8, 16, kv_dtype="fp8", seed=13), [16, 5, 47]),
]


@pytest.mark.parametrize("w,lens", SMALL, ids=[w.name for w, _ in SMALL])
def test_bruteforce_matches_reference(w, lens):
    inp = make_inputs(w, lengths=lens)
    ref = run_ref(inp)
    bf = run_ref(inp, fn=attention_bruteforce)
    assert np.all(np.isfinite(ref))
    np.testing.assert_allclose(ref, bf, rtol=0, atol=1e-12)


def test_selected_matches_full():
    inp = make_inputs(Workload("sel", 3, 8, 2, 16, 16, seed=5), lengths=[20, 70, 3])
    full = run_ref(inp)
    pairs = [(0, 0), (1, 5), (2, 7), (1, 3)]
    sel = run_ref(inp, fn=attention_selected, pairs=pairs)
    for p in pairs:
        np.testing.assert_allclose(sel[p], full[p], rtol=0, atol=1e-14)


def test_single_token_returns_its_value():
    w = Workload("len1", 4, 8, 2, 32, 16, seed=21)
    inp = make_inputs(w, lengths=[1, 1, 1, 1])
    out = run_ref(inp)
    for b in range(4):
        v = decode_kv(gather_request(inp["v_pages"], inp["block_table"][b], 1, 16), "bf16")
        for h in range(8):
            assert np.array_equal(out[b, h], v[0, h // 4])


def test_constant_values_give_that_value():
    w = Workload("constv", 2, 4, 2, 16, 16, seed=22)
    inp = make_inputs(w, lengths=[37, 64], poison=False)
    vp = inp["v_pages"]
    row = vp[0, :, 0, :].copy()
    vp[:] = row[None, :, None, :]
    out = run_ref(inp)
    v = decode_kv(row, "bf16")
    for b in range(2):
        for h in range(4):
            np.testing.assert_allclose(out[b, h], v[h // 2], rtol=1e-14, atol=0)


def test_zero_query_gives_mean_value():
    w = Workload("q0", 2, 4, 2, 16, 16, seed=23)
    inp = make_inputs(w, lengths=[29, 100])
    q = np.zeros((2, 4, 16))
    out = run_ref(inp, q=q)
    for b, L in enumerate([29, 100]):
        v = decode_kv(gather_request(inp["v_pages"], inp["block_table"][b], L, 16), "bf16")
        for h in range(4):
            np.testing.assert_allclose(out[b, h], v[:, h // 2].mean(axis=0), rtol=0, atol=1e-14)


def test_dominant_key():
    w = Workload("dom", 1, 2, 1, 16, 16, seed=24)
    L, tstar = 200, 137
    inp = make_inputs(w, lengths=[L], poison=False)
    kp = inp["k_pages"]
    kp[:] = np.uint16(0x3C23)                       # bf16 0.00996...
    page = inp["block_table"][0][tstar // 16]
    kp[page, 0, tstar % 16, 0] = np.uint16(0x4480)  # bf16 1024
    q = np.zeros((1, 2, 16))
    q[0, :, 0] = 1.0
    out = run_ref(inp, q=q)
    v = decode_kv(inp["v_pages"][page, 0, tstar % 16], "bf16")
    # every other score is lower by (1024 - 0.00996) / 4 > 50
    bound = L * math.exp(-50) * 10
    for h in range(2):
        np.testing.assert_allclose(out[0, h], v, rtol=0, atol=bound)


def test_score_shift_invariance():
    w = Workload("shift", 2, 4, 2, 16, 16, seed=25)
    inp = make_inputs(w, lengths=[45, 80], poison=False)
    inp["k_pages"][:, :, :, 3] = np.uint16(0x3F80)  # K[..., 3] = 1 for every token
    q = oa.bf16_to_f64(inp["q"])
    a = run_ref(inp, q=q)
    q2 = q.copy()
    q2[:, :, 3] += 2.5                              # every score moves by the same amount
    b = run_ref(inp, q=q2)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


def _sdpa(inp, expand_gqa):
    q = oa.bf16_to_f64(inp["q"])
    B, Hq, D = q.shape
    Hkv = inp["k_pages"].shape[1]
    ps = inp["k_pages"].shape[2]
    out = np.zeros_like(q)
    for b, L in enumerate(inp["seq_lens"].tolist()):
        k = decode_kv(gather_request(inp["k_pages"], inp["block_table"][b], L, ps), "bf16")
        v = decode_kv(gather_request(inp["v_pages"], inp["block_table"][b], L, ps), "bf16")
        kt = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2)))[None]   # [1, Hkv, L, D]
        vt = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2)))[None]
        if expand_gqa:
            kt = kt.repeat_interleave(Hq // Hkv, dim=1)
            vt = vt.repeat_interleave(Hq // Hkv, dim=1)
        qt = torch.from_numpy(q[b])[None, :, None, :]                              # [1, Hq, 1, D]
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=float(inp["sm_scale"]))
        out[b] = o[0, :, 0, :].numpy()
    return out


def test_matches_torch_sdpa_mha():
    w = Workload("sdpa", 3, 4, 4, 32, 16, placement="contiguous", seed=26)
    inp = make_inputs(w, lengths=[5, 64, 130])
    np.testing.assert_allclose(run_ref(inp), _sdpa(inp, False), rtol=0, atol=1e-12)


def test_matches_torch_sdpa_gqa_expanded():
    w = Workload("sdpa_gqa", 3, 8, 2, 32, 16, seed=27)
    inp = make_inputs(w, lengths=[9, 64, 200])
    np.testing.assert_allclose(run_ref(inp), _sdpa(inp, True), rtol=0, atol=1e-12)


def test_page_permutation_invariance():
    w = Workload("perm", 4, 8, 2, 16, 16, seed=28)
    inp = make_inputs(w, lengths=[33, 1, 90, 16])
    a = run_ref(inp)
    n = inp["k_pages"].shape[0]
    pi = np.random.default_rng(0).permutation(n)        # new physical id of page p
    inv = np.argsort(pi)
    inp2 = dict(inp)
    inp2["k_pages"] = inp["k_pages"][inv]
    inp2["v_pages"] = inp["v_pages"][inv]
    bt = inp["block_table"].copy()
    bt[bt >= 0] = pi[bt[bt >= 0]]
    inp2["block_table"] = bt
    assert np.array_equal(a, run_ref(inp2))


PLANS = [("dyn", 1, 1), ("dyn", 16, 3), ("dyn", 16, 64), ("dyn", 64, 5), ("dyn", 7, 11),
         ("static", 1, None), ("static", 2, None), ("static", 7, None)]


@pytest.mark.parametrize("kind,a,b", PLANS)
def test_split_merge_equals_unsplit(kind, a, b):
    w = Workload("split", 5, 8, 2, 16, 16, seed=29)
    lens = [1, 17, 64, 150, 333]
    inp = make_inputs(w, lengths=lens)
    plan = plan_dynamic(lens, a, b) if kind == "dyn" else plan_static(lens, a)
    ref = run_ref(inp)
    sm = run_ref(inp, fn=split_merge_reference, plan=plan)
    np.testing.assert_allclose(sm, ref, rtol=0, atol=1e-12)


def test_split_merge_fp8():
    w = Workload("split8", 3, 4, 2, 16, 16, kv_dtype="fp8", seed=30)
    lens = [100, 7, 64]
    inp = make_inputs(w, lengths=lens)
    ref = run_ref(inp)
    sm = run_ref(inp, fn=split_merge_reference, plan=plan_dynamic(lens, 16, 6))
    np.testing.assert_allclose(sm, ref, rtol=0, atol=1e-12)


# --- planted mistakes: each must be caught by one of the pins above --------

def test_planted_wrong_head_mapping_is_caught(monkeypatch):
    w = Workload("sdpa_gqa", 3, 8, 2, 32, 16, seed=27)
    inp = make_inputs(w, lengths=[9, 64, 200])
    good = _sdpa(inp, True)
    monkeypatch.setattr(oa, "_kv_head", lambda h, hq, hkv: h % hkv)
    assert not np.allclose(run_ref(inp), good, atol=1e-3)


def test_planted_missing_scale_is_caught():
    w = Workload("sdpa", 3, 4, 4, 32, 16, placement="contiguous", seed=26)
    inp = make_inputs(w, lengths=[5, 64, 130])
    good = _sdpa(inp, False)
    q64 = oa.bf16_to_f64(inp["q"])
    bad = attention_reference(q64, inp["k_pages"], inp["v_pages"], inp["block_table"],
                              inp["seq_lens"], "bf16", 1.0)
    assert not np.allclose(bad, good, atol=1e-3)


def test_planted_wrong_gather_is_caught(monkeypatch):
    w = Workload("mha", 3, 4, 4, 16, 16, seed=11)
    inp = make_inputs(w, lengths=[1, 33, 50])
    bf = run_ref(inp, fn=attention_bruteforce)

    def bad_gather(pages, row, length, ps):
        n = (length + ps - 1) // ps
        g = pages[np.asarray(row[:n], dtype=np.int64)]          # [n, Hkv, ps, D]
        # mistake: reshape without moving the page-row axis next to the page axis
        return g.reshape(n * ps, g.shape[1], g.shape[3])[:length]

    monkeypatch.setattr(oa, "gather_request", bad_gather)
    with np.errstate(invalid="ignore"):
        bad = run_ref(inp)
    assert not np.allclose(bad, bf, atol=1e-3, equal_nan=False)

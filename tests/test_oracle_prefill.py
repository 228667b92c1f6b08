"""Pins for the multi-token (prefill) oracle and its row-block rule (CPU).

Checked against: the decode oracle when every request brings one query (a
reduction to a pinned function); a pure-Python brute force with its own page
lookups and causal limit; causality (changing cache tokens after a row's
position leaves that row unchanged and changes a later row); closed forms of
a full prefill (row 0 sees only token 0, so it returns V[0]; the last row is
decode over the whole cache); and the hand-worked rows and plan in
tests/golden/prefill_rows.txt.  Planted mistakes (a causal limit one token
off either way) must be caught.
"""

import math
import os

import numpy as np
import pytest

import oracle
import oracle.prefill as op
from load_balanced_split_step_amd.workloads import Workload, make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "prefill_rows.txt")


def run(inp, fn=op.prefill_reference):
    return fn(oracle.bf16_to_f64(inp["q"]), inp["k_pages"], inp["v_pages"], inp["block_table"],
              inp["seq_lens"], inp["q_lens"], inp["kv_dtype"], float(inp["sm_scale"]),
              k_scale=float(inp["k_scale"]), v_scale=float(inp["v_scale"]),
              scale_mode=inp["scale_mode"], k_scales=inp["k_scales"], v_scales=inp["v_scales"])


W = Workload("pf", 3, 8, 2, 16, 16, seed=60)


def brute(inp):
    """Pure-Python loops: per packed row, its own page lookups and limit."""
    qf = oracle.bf16_to_f64(inp["q"]).tolist()
    kd = oracle.decode_kv(inp["k_pages"], inp["kv_dtype"], float(inp["k_scale"])).tolist()
    vd = oracle.decode_kv(inp["v_pages"], inp["kv_dtype"], float(inp["v_scale"])).tolist()
    bt = inp["block_table"].tolist()
    ps = inp["k_pages"].shape[2]
    Hq, Hkv, D = len(qf[0]), inp["k_pages"].shape[1], len(qf[0][0])
    out = []
    row = 0
    for b, (n, L) in enumerate(zip(inp["q_lens"].tolist(), inp["seq_lens"].tolist())):
        for r in range(n):
            pos = L - n + r
            heads = []
            for h in range(Hq):
                kvh = (h * Hkv) // Hq
                sc = [float(inp["sm_scale"]) * math.fsum(
                    qf[row][h][d] * kd[bt[b][t // ps]][kvh][t % ps][d] for d in range(D))
                    for t in range(pos + 1)]
                m = max(sc)
                w = [math.exp(x - m) for x in sc]
                z = math.fsum(w)
                heads.append([math.fsum(w[t] * vd[bt[b][t // ps]][kvh][t % ps][d]
                                        for t in range(pos + 1)) / z for d in range(D)])
            out.append(heads)
            row += 1
    return np.array(out)


def test_single_query_equals_decode():
    inp = make_inputs(W, lengths=[40, 7, 100], q_lens=[1, 1, 1])
    dec = oracle.attention_reference(oracle.bf16_to_f64(inp["q"]), inp["k_pages"], inp["v_pages"],
                                     inp["block_table"], inp["seq_lens"], "bf16",
                                     float(inp["sm_scale"]))
    np.testing.assert_allclose(run(inp), dec, rtol=0, atol=1e-12)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_bruteforce(kv):
    inp = make_inputs(W.with_(kv_dtype=kv), lengths=[20, 5, 33], q_lens=[4, 5, 2])
    np.testing.assert_allclose(run(inp), brute(inp), rtol=0, atol=1e-12)


def test_causality():
    inp = make_inputs(W, lengths=[50, 30, 64], q_lens=[6, 3, 10], poison=False)
    base = run(inp)
    # change every cache token of request 0 after position 46 (its row 2)
    ps = inp["k_pages"].shape[2]
    L, n = 50, 6
    pos_r2 = L - n + 2
    kp = inp["k_pages"].copy()
    vp = inp["v_pages"].copy()
    for t in range(pos_r2 + 1, L):
        pg = inp["block_table"][0][t // ps]
        kp[pg, :, t % ps, :] ^= np.uint16(0x0140)
        vp[pg, :, t % ps, :] ^= np.uint16(0x0140)
    out = run(dict(inp, k_pages=kp, v_pages=vp))
    np.testing.assert_array_equal(out[:3], base[:3])         # rows 0..2 of request 0
    assert not np.allclose(out[3], base[3])                  # row 3 sees the change
    np.testing.assert_array_equal(out[6:], base[6:])         # other requests untouched


def test_full_prefill_closed_forms():
    inp = make_inputs(W, lengths=[24, 17, 5], q_lens=[24, 17, 5])
    out = run(inp)
    off = oracle.q_offsets(inp["q_lens"])
    ps = inp["k_pages"].shape[2]
    Hq, Hkv = 8, 2
    for b in range(3):
        v0 = oracle.bf16_to_f64(inp["v_pages"][inp["block_table"][b][0], :, 0, :])   # [Hkv, D]
        for h in range(Hq):
            np.testing.assert_array_equal(out[off[b], h], v0[(h * Hkv) // Hq])
    last = [off[b + 1] - 1 for b in range(3)]
    dec = oracle.attention_reference(oracle.bf16_to_f64(inp["q"])[last], inp["k_pages"],
                                     inp["v_pages"], inp["block_table"], inp["seq_lens"], "bf16",
                                     float(inp["sm_scale"]))
    np.testing.assert_allclose(out[last], dec, rtol=0, atol=1e-12)


def _golden():
    g = {"row": [], "item": []}
    for line in open(GOLDEN):
        if not line.strip() or line.startswith("#"):
            continue
        k, *v = line.split()
        if k in ("row", "item"):
            g[k].append(tuple(int(x) for x in v))
        elif k == "plan":
            g[k] = v
        else:
            g[k] = [int(x) for x in v]
    return g


def test_rows_and_plan_golden():
    g = _golden()
    rows, ext = op.prefill_rows(g["q_lens"], g["kv_lens"], g["rows_per_block"][0])
    assert rows == g["row"] and ext == g["extents"]
    p = oracle.plan_dynamic(ext, int(g["plan"][1]), int(g["plan"][2]))
    assert p.to_list()[:8] == g["header"]
    assert list(p.wg_ptr) == g["wg_ptr"]
    assert [tuple(x) for x in p.items] == g["item"]
    assert list(p.req_part_ptr) == g["req_part_ptr"]


def test_rows_properties():
    rng = np.random.default_rng(4)
    for _ in range(200):
        B = int(rng.integers(1, 12))
        kv = rng.integers(1, 300, size=B)
        ql = np.minimum(rng.integers(1, 60, size=B), kv)
        qb = int(rng.choice([1, 2, 4, 16]))
        rows, ext = op.prefill_rows(ql, kv, qb)
        seen = []
        for (b, q0, nq, pos0), e in zip(rows, ext):
            assert 1 <= nq <= qb and e == pos0 + nq
            seen += [(b, q0 + r, pos0 + r) for r in range(nq)]
        off = oracle.q_offsets(ql)
        want = [(b, off[b] + r, kv[b] - ql[b] + r) for b in range(B) for r in range(ql[b])]
        assert seen == want


@pytest.mark.parametrize("shift", [-1, 1])
def test_planted_causal_limit_is_caught(monkeypatch, shift):
    inp = make_inputs(W, lengths=[20, 5, 33], q_lens=[4, 5, 2])
    good = brute(inp)
    real_gather = op.gather_request

    def shifted(pages, row, length, ps):
        return real_gather(pages, row, length, ps)

    # plant: attend to tokens 0..pos+shift by moving kv_len
    bad_lens = inp["seq_lens"] + shift
    with np.errstate(invalid="ignore"):
        try:
            bad = op.prefill_reference(oracle.bf16_to_f64(inp["q"]), inp["k_pages"], inp["v_pages"],
                                       inp["block_table"], bad_lens, inp["q_lens"], "bf16",
                                       float(inp["sm_scale"]))
        except (IndexError, ValueError):
            return                                            # caught by construction
    assert not np.allclose(bad, good, atol=1e-3, equal_nan=False)

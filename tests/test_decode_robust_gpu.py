"""Decode under the conditions a serving loop brings: lengths that changed
after the plan was built, requests sharing prefix pages, batch membership
changing between steps, and an exactly-once coverage count of the tiles.

The pages ask kernels to survive changing sequence lengths and boundary
shapes, and name prefix caching and continuous batching among the serving
features results depend on (remio.ai page, section "Lo que la afirmación de
un 48,8 % de TPOT no demuestra"); the tiles are rebuilt as lengths change
(same page, section "Por qué Tencent HPC importa para el serving de modelos
en línea").  Bar: the fp64 oracle at the device lengths, 2e-2 (bf16 cache)
or 6e-2 (fp8 cache) max-abs.
"""

import numpy as np
import pytest
import torch

import load_balanced_split_step_amd.hda as hda
import oracle
from load_balanced_split_step_amd.workloads import CONFIGS, Workload, make_inputs
from tests.gpu_util import TOL, max_err, need_gpu, oracle_out, scale_kw

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _bf16_bits(x):
    """float values -> bf16 bit patterns (uint16), torch's nearest-even cast."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _oracle_at(inp, lens, q=None, block_table=None):
    return oracle.attention_reference(
        oracle.bf16_to_f64(inp["q"] if q is None else q), inp["k_pages"], inp["v_pages"],
        inp["block_table"] if block_table is None else block_table, lens, inp["kv_dtype"],
        float(inp["sm_scale"]), **scale_kw(inp))


STALE = {
    "bf16": (Workload("stale", 7, 16, 2, 128, 32, seed=81), [5000, 1000, 999, 64, 40, 2049, 700]),
    "fp8_page": (Workload("stale8", 6, 16, 4, 64, 16, kv_dtype="fp8", kv_scale="page",
                          head_scale=True, seed=82), [300, 47, 1, 900, 33, 128]),
}


@pytest.mark.parametrize("name", list(STALE))
def test_stale_plan_built_for_longer_lengths(name):
    """A plan built for longer lengths than the device holds (lengths rolled
    back, e.g. rejected draft tokens): the rows between the two lengths hold
    real, stale keys and values.  Every path masks them -- the output is the
    oracle's at the device lengths -- and reports HDA_CHECK_PAST_LEN."""
    w, lens_plan = STALE[name]
    lens_plan = np.array(lens_plan, np.int32)
    inp = make_inputs(w, lengths=lens_plan)            # the cache holds the longer lengths
    lens_dev = np.maximum(1, lens_plan - np.array([37, 1, 0, 63, 39, 500, 1][:w.batch], np.int32))
    ref = _oracle_at(inp, lens_dev)
    dev = hda.DeviceBatch.from_inputs(inp)
    dev.t["seq_lens"].copy_(torch.from_numpy(lens_dev))
    tol = TOL[w.kv_dtype]
    plans = [("dyn", hda.hda_plan(lens_plan, 64, 13)), ("dyn-tile16", hda.hda_plan(lens_plan, 16, 97)),
             ("static-3", hda.hda_plan_static(lens_plan, 3))]
    for pname, plan in plans:
        for upload in ("copy", "bench"):
            if upload == "bench" and plan.size > hda.HDA_PLAN_ARG_INTS:
                continue
            out = dev.decode(plan, upload=upload)
            torch.cuda.synchronize()
            err = max_err(out, ref)
            bits = dev.check(plan)
            print(f"{name} {pname} {upload}: max err {err:.3e}, check bits {bits}", flush=True)
            assert err <= tol, (pname, upload, err)
            assert bits == hda.HDA_CHECK_PAST_LEN, (pname, upload, bits)
    # the same plan at the lengths it was built for is clean
    dev.t["seq_lens"].copy_(torch.from_numpy(lens_plan))
    dev.decode(plans[0][1])
    assert dev.check(plans[0][1]) == 0


def test_stale_plan_native_fp8():
    w = CONFIGS["fp8"].with_(name="stale_n", batch=6, prologue=False, len_range=(100, 2000))
    inp = make_inputs(w)
    lens_plan = inp["seq_lens"]
    lens_dev = np.maximum(1, lens_plan - np.array([65, 0, 1, 64, 99, 3], np.int32))
    exact = _oracle_at(inp, lens_dev)
    dev = hda.DeviceBatch.from_inputs(inp, math="fp8")
    dev.t["seq_lens"].copy_(torch.from_numpy(lens_dev))
    plan = hda.hda_plan(lens_plan, 128, 11)
    out = dev.decode(plan)
    torch.cuda.synchronize()
    err = max_err(out, exact)
    print(f"native fp8, stale plan: max err {err:.3e}", flush=True)
    assert err <= TOL["fp8"]
    assert dev.check(plan) == hda.HDA_CHECK_PAST_LEN


def test_stale_plan_built_for_shorter_lengths():
    """A plan built for shorter lengths: the tokens past the plan's end are
    not attended (the kernel cannot know of them beyond the check), the
    output is the oracle's at the plan's lengths, and HDA_CHECK_SHORT is
    reported; with mixed errors both bits are."""
    w, lens = STALE["bf16"]
    lens = np.array(lens, np.int32)
    inp = make_inputs(w, lengths=lens)
    dev = hda.DeviceBatch.from_inputs(inp)
    short = lens.copy()
    short[[0, 3]] -= [100, 10]
    plan = hda.hda_plan(short, 64, 9)
    out = dev.decode(plan)
    torch.cuda.synchronize()
    assert max_err(out, _oracle_at(inp, short)) <= TOL["bf16"]
    assert dev.check(plan) == hda.HDA_CHECK_SHORT
    mixed = lens.copy()
    mixed[0] -= 5
    mixed[1] += 3
    plan = hda.hda_plan(mixed, 64, 9)
    dev.decode(plan)
    assert dev.check(plan) == hda.HDA_CHECK_SHORT | hda.HDA_CHECK_PAST_LEN


def _expected_visits(block_table, lens, n_pages, ps, n_kv_heads):
    e = np.zeros((n_pages, ps, n_kv_heads), np.int32)
    for b, L in enumerate(np.asarray(lens).tolist()):
        t = np.arange(L)
        np.add.at(e, (block_table[b][t // ps], t % ps), 1)
    return e


COVER = {
    "tiny": (CONFIGS["tiny"], None, "bf16"),
    "extreme_s": (CONFIGS["extreme"].with_(name="cov_x", batch=6), [9000, 1000, 17, 1, 4096, 65],
                  "bf16"),
    "fp8_page_s": (CONFIGS["fp8_page"].with_(name="cov_p", batch=7, len_range=(1, 3000),
                                             prologue=False), None, "bf16"),
    "native_fp8": (CONFIGS["fp8"].with_(name="cov_n", batch=7, len_range=(1, 3000),
                                        prologue=False), None, "fp8"),
    "d64_page16": (Workload("cov_d64", 5, 8, 2, 64, 16, seed=83), [16, 15, 33, 1000, 2], "bf16"),
}


@pytest.mark.parametrize("name", list(COVER))
def test_coverage_every_token_once(name):
    """The coverage-counting launch: every row below each request's length
    is scored exactly once per kv head, nothing else is, and the outputs
    stay within the bar."""
    w, lens, math_ = COVER[name]
    inp = make_inputs(w, lengths=lens)
    L = inp["seq_lens"]
    dev = hda.DeviceBatch.from_inputs(inp, math=math_)
    ps = w.page_size
    expect = _expected_visits(inp["block_table"], L, inp["k_pages"].shape[0], ps, w.n_kv_heads)
    ref = oracle_out(inp)
    T = int(sum(-(-int(x) // 16) for x in L))
    for pname, plan in [("default", hda.hda_plan(L, *hda.launch_config(L, w.n_kv_heads))),
                        ("tile16", hda.hda_plan(L, 16, 37)), ("wide", hda.hda_plan(L, 32, T + 5)),
                        ("one-wg", hda.hda_plan(L, 64, 1)), ("static-4", hda.hda_plan_static(L, 4))]:
        out, visits = dev.coverage(plan)
        torch.cuda.synchronize()
        got = visits.cpu().numpy()
        assert np.array_equal(got, expect), (pname, int(np.abs(got - expect).sum()))
        err = max_err(out, ref)
        print(f"{name} {pname}: coverage exact, max err {err:.3e}", flush=True)
        if math_ == "bf16":
            assert err <= TOL[w.kv_dtype], (pname, err)


def _share_prefix(inp, n_shared_pages, members):
    """Block table where requests `members` read the first n_shared_pages
    physical pages of members[0] (a common prompt prefix in a prefix cache)."""
    bt = inp["block_table"].copy()
    src = members[0]
    for b in members[1:]:
        bt[b, :n_shared_pages] = bt[src, :n_shared_pages]
    return bt


def test_shared_prefix_pages():
    """Requests whose block tables point at the same physical prefix pages:
    each attends the shared rows as its own; coverage counts a shared row
    once per request that reads it."""
    w = Workload("prefix", 6, 16, 2, 128, 32, seed=84)
    lens = np.array([4000, 3000, 1100, 960, 5000, 129], np.int32)
    inp = make_inputs(w, lengths=lens)
    bt = _share_prefix(inp, 30, [0, 1, 2, 3, 4])     # 960 tokens = 30 pages of 32
    inp2 = dict(inp, block_table=bt)
    ref = oracle_out(inp2)
    dev = hda.DeviceBatch.from_inputs(inp2)
    for plan in (hda.hda_plan(lens, *hda.launch_config(lens, w.n_kv_heads)),
                 hda.hda_plan(lens, 32, 50), hda.hda_plan_static(lens, 2)):
        out = dev.decode(plan, upload="bench" if plan.size <= hda.HDA_PLAN_ARG_INTS else "copy")
        torch.cuda.synchronize()
        assert max_err(out, ref) <= TOL["bf16"]
        _, visits = dev.coverage(plan)
        expect = _expected_visits(bt, lens, inp["k_pages"].shape[0], w.page_size, w.n_kv_heads)
        assert expect.max() == 5
        assert np.array_equal(visits.cpu().numpy(), expect)
    # request 3 is exactly the shared prefix: its output equals request 0's
    # attention over that prefix with request 3's query
    lens3 = lens.copy()
    lens3[0] = 960
    q = inp["q"].copy()
    q[0] = q[3]
    ref0 = _oracle_at(inp2, lens3, q=q)
    assert float(np.abs(ref0[0] - ref[3]).max()) < 1e-12
    assert max_err(out[3:4], ref[3:4]) <= TOL["bf16"]


def test_continuous_batching_membership_changes():
    """A serving loop: requests join and leave between steps, the others
    grow by one token per step; every step builds a new batch (block-table
    rows, lengths, q) over the same page pool, re-plans, and matches the
    oracle through both plan paths."""
    w = Workload("cb", 7, 16, 2, 128, 32, seed=85)
    full = np.array([3000, 1500, 700, 64, 2500, 40, 1200], np.int32)   # lengths at the last step
    inp = make_inputs(w, lengths=full)
    dev = hda.DeviceBatch.from_inputs(inp)
    rng = np.random.default_rng(86)
    schedule = [[0, 1, 2], [0, 1, 2, 3], [0, 2, 3, 4], [0, 4], [4, 5, 6, 0, 2], [6, 5, 4]]
    n_steps = len(schedule)
    for s, members in enumerate(schedule):
        idx = np.array(members)
        lens = (full[idx] - (n_steps - 1 - s)).astype(np.int32)        # one more token per step
        q = _bf16_bits(rng.standard_normal((len(idx), w.n_q_heads, w.head_dim)))
        bt = inp["block_table"][idx]
        ref = _oracle_at(inp, lens, q=q, block_table=bt)
        t_q = torch.from_numpy(q.view(np.int16)).cuda()
        t_bt = torch.from_numpy(np.ascontiguousarray(bt)).cuda()
        t_len = torch.from_numpy(lens).cuda()
        kw = dict(dev.kw, batch=len(idx))
        for upload in ("bench", "copy"):
            plan = hda.hda_plan(lens, *hda.launch_config(lens, w.n_kv_heads))
            p = hda.hda_params(**kw)
            need = hda.hda_workspace_bytes(plan, w.n_q_heads, w.n_kv_heads, w.head_dim)
            ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda:0")
            p.workspace, p.workspace_bytes = ws.data_ptr(), ws.numel()
            out = torch.empty((len(idx), w.n_q_heads, w.head_dim), dtype=torch.float32,
                              device="cuda:0")
            pd = None if upload == "bench" else torch.from_numpy(plan).cuda()
            hda.hda_decode(p, t_q, dev.t["k_pages"], dev.t["v_pages"], t_bt, t_len, plan, pd, out)
            torch.cuda.synchronize()
            err = max_err(out, ref)
            print(f"step {s} members {members} ({upload}): max err {err:.3e}", flush=True)
            assert err <= TOL["bf16"]
            assert hda.hda_decode_check(p, int(plan[3])) == 0


def test_prefill_stale_lengths_report_past_len():
    """hda_prefill with device cache lengths shorter than the ones its row
    blocks were planned for: no token at or past a device length is scored
    (outputs stay finite: the rows past each length hold NaN), and the check
    words report HDA_CHECK_PAST_LEN; at the planned lengths they are clear."""
    w = Workload("pf_stale", 4, 16, 2, 128, 32, seed=87)
    inp = make_inputs(w, lengths=[700, 1500, 96, 3000], q_lens=[5, 40, 17, 64])
    dev = hda.DeviceBatch.from_inputs(inp)
    rows, plan = dev.prefill_plan(inp["q_lens"])
    dev.prefill(rows, plan)
    p = dev.prefill_params(plan)
    assert hda.hda_decode_check(p, int(plan[3])) == 0
    shorter = (inp["seq_lens"] - np.array([3, 0, 20, 1], np.int32)).astype(np.int32)
    dev.t["seq_lens"].copy_(torch.from_numpy(shorter))
    out = dev.prefill(rows, plan)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    assert hda.hda_decode_check(p, int(plan[3])) == hda.HDA_CHECK_PAST_LEN

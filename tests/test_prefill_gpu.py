"""GPU parity of multi-token attention (hda_prefill) against the fp64 oracle.

Row blocks of 1, 2, 4, 8 or 16 tiles of 16 / group query rows (the column
kernel and the LDS-shared shapes: 4 waves of one tile, 8 of one, 8 of two,
and 16 of one over an fp8 cache without per-page factors) go through the
decode tile planner;
every block of an item loads its next stage while multiplying the current
one, the last stage of an item the next item's first; checked element by
element at
sizes the oracle finishes in seconds (ragged q lengths, partial blocks whose
last tiles are idle, blocks split over workgroups, plan tiles not aligned to
chunks, every group size the kernel takes), one query per request bitwise
equal to the decode path, score patterns that move the softmax's running
maximum again and again (keys growing along the sequence, a late key that
dominates), and the full-size speculative-check and chunked workloads on
sampled rows.
Bar: 2e-2 (bf16 cache), 6e-2 (fp8 cache) max-abs error.
"""

import numpy as np
import pytest
import torch

import load_balanced_split_step_amd.hda as hda
import oracle
from load_balanced_split_step_amd.workloads import CONFIGS, Workload, _bf16_bits, make_inputs
from tests.gpu_util import TOL, need_gpu, scale_kw, max_err

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def ref_prefill(inp):
    return oracle.prefill_reference(oracle.bf16_to_f64(inp["q"]), inp["k_pages"], inp["v_pages"],
                                    inp["block_table"], inp["seq_lens"], inp["q_lens"],
                                    inp["kv_dtype"], float(inp["sm_scale"]), **scale_kw(inp))


CASES = {
    "tiny_pf": (CONFIGS["tiny"].with_(name="tiny_pf", q_len_range=(1, 20)), None, None),
    "spec_s": (CONFIGS["specdec"].with_(name="spec_s", batch=8, lengths=None,
                                        q_lens=(4,) * 8), [16384] + [1000] * 7, None),
    "chunk_s": (CONFIGS["chunked"].with_(name="chunk_s", batch=6, len_range=(200, 3000),
                                         q_len_range=(1, 70)), None, None),
    "full_s": (Workload("full_s", 4, 16, 4, 128, 16, seed=80), [1, 33, 130, 257], [1, 33, 130, 257]),
    "fp8_page_pf": (CONFIGS["fp8_page"].with_(name="fp8_page_pf", batch=6, len_range=(100, 2500),
                                              prologue=False, q_len_range=(1, 40)), None, None),
    "fp8_d64_tensor": (Workload("fp8_d64_tensor", 4, 16, 4, 64, 16, kv_dtype="fp8", seed=83),
                       [40, 700, 129, 2000], [7, 33, 1, 64]),
    "fp8_head_pf": (CONFIGS["fp8_page"].with_(name="fp8_head_pf", batch=5, len_range=(100, 2000),
                                              prologue=False, kv_scale="head",
                                              q_len_range=(1, 50)), None, None),
    "g16": (Workload("g16", 3, 32, 2, 128, 64, seed=81), [700, 90, 2000], [20, 3, 33]),
    "g1": (Workload("g1", 3, 4, 4, 64, 32, seed=82), [300, 64, 65], [40, 64, 1]),
    "ps128": (Workload("ps128", 4, 16, 2, 128, 128, seed=85), [1000, 129, 384, 2100],
              [50, 3, 64, 17]),
    "ps1024_fp8": (Workload("ps1024_fp8", 3, 16, 2, 128, 1024, kv_dtype="fp8", seed=86),
                   [1500, 1024, 3000], [20, 64, 5]),
}


@pytest.mark.parametrize("tiles", [1, 2, 4, 8, 16],
                         ids=["1tile-columns", "2tiles-lds4", "4tiles-lds4", "8tiles-lds8",
                              "16tiles-lds8x2-fp8-16x1"])
@pytest.mark.parametrize("name", list(CASES))
def test_prefill_parity(name, tiles):
    """Blocks of 1 tile of 16/g rows (decode column shape), or of 2 to 16
    tiles with each K/V chunk loaded once into LDS (4 waves of one tile, 8 of
    one, 8 of two) and multiplied by every tile."""
    w, lens, qlens = CASES[name]
    inp = make_inputs(w, lengths=lens, q_lens=qlens)
    ref = ref_prefill(inp)
    dev = hda.DeviceBatch.from_inputs(inp)
    qb = hda.hda_prefill_rows_per_block(w.n_q_heads, w.n_kv_heads) * tiles
    rows, row_lens = hda.hda_prefill_rows(inp["q_lens"], inp["seq_lens"], qb)
    plans = [("default", dev.prefill_plan(inp["q_lens"], tiles=tiles)[1])]
    for tl, W in [(64, 7), (100, 13), (16, 300), (512, 2)]:
        plans.append((f"dyn-{tl}-{W}", hda.hda_plan(row_lens, tl, W)))
    plans.append(("static-3", hda.hda_plan_static(row_lens, 3)))
    tol = TOL[w.kv_dtype]
    for pname, plan in plans:
        out = dev.prefill(rows, plan)
        torch.cuda.synchronize()
        err = max_err(out, ref)
        print(f"{name} {pname} {tiles} tiles: {len(rows)} blocks, "
              f"P={int(plan[6])}, max err {err:.3e}", flush=True)
        assert err <= tol, (name, pname, err)


def _reshape_keys(inp, rate, jump):
    """Scale the cached key of token t of every request by 1 + rate * t, and
    the key of its last cached token before the new rows by `jump` more
    (bf16, round to nearest even; the poisoned slots past each length stay
    as they are): the scores grow along the sequence, so the running maximum
    keeps moving, and the late key dominates the columns it aligns with."""
    w = inp["workload"]
    ps = w.page_size
    k = inp["k_pages"].copy()
    for b, L in enumerate(inp["seq_lens"]):
        L = int(L)
        t_jump = L - int(inp["q_lens"][b]) - 1
        for p in range(-(-L // ps)):
            pg = int(inp["block_table"][b, p])
            n = min(ps, L - p * ps)
            t = p * ps + np.arange(n)
            f = (1.0 + rate * t) * np.where(t == t_jump, jump, 1.0)
            rows = oracle.bf16_to_f64(k[pg, :, :n, :]) * f[None, :, None]
            k[pg, :, :n, :] = _bf16_bits(rows.astype(np.float32))
    return dict(inp, k_pages=k)


@pytest.mark.parametrize("tiles", [1, 2, 4, 16], ids=["1tile", "2tiles", "4tiles", "16tiles"])
@pytest.mark.parametrize("pattern", ["growth", "jump"])
def test_prefill_moving_maximum(pattern, tiles):
    """Keys scaled up along the sequence (x 1 + t / 40: the column maxima
    pass the softmax's reference by more than 2^8 again and again), or in
    addition one late key x 40; bf16 cache, the default plan and a fine one."""
    w = CONFIGS["chunked"].with_(name="moving_max", batch=4, len_range=(300, 2500),
                                 q_len_range=(1, 40), seed=84)
    inp = _reshape_keys(make_inputs(w), 1.0 / 40, 40.0 if pattern == "jump" else 1.0)
    ref = ref_prefill(inp)
    dev = hda.DeviceBatch.from_inputs(inp)
    qb = hda.hda_prefill_rows_per_block(w.n_q_heads, w.n_kv_heads) * tiles
    rows, row_lens = hda.hda_prefill_rows(inp["q_lens"], inp["seq_lens"], qb)
    for pname, plan in [("default", dev.prefill_plan(inp["q_lens"], tiles=tiles)[1]),
                        ("dyn-64-11", hda.hda_plan(row_lens, 64, 11))]:
        out = dev.prefill(rows, plan)
        torch.cuda.synchronize()
        err = max_err(out, ref)
        print(f"{pattern} {pname} {tiles} tiles: max err {err:.3e}", flush=True)
        assert err <= TOL["bf16"], (pattern, pname, err)


def test_single_query_rows_bitwise_equal_decode():
    w = CONFIGS["extreme"].with_(name="pf1", batch=8)
    lens = [9000] + [700] * 7
    inp = make_inputs(w, lengths=lens, q_lens=[1] * 8)
    dev = hda.DeviceBatch.from_inputs(inp)
    rows, row_lens = hda.hda_prefill_rows(inp["q_lens"], inp["seq_lens"], 2)
    assert np.array_equal(row_lens, inp["seq_lens"])
    for tl, W in [(128, 24), (64, 5)]:
        plan = hda.hda_plan(row_lens, tl, W)
        a = dev.prefill(rows, plan)
        b = dev.decode(plan)
        torch.cuda.synchronize()
        assert torch.equal(a, b), (tl, W)


def test_specdec_full_size_sampled():
    w = CONFIGS["specdec"]
    inp = make_inputs(w)
    dev = hda.DeviceBatch.from_inputs(inp)
    rows, plan = dev.prefill_plan(inp["q_lens"])
    out = dev.prefill(rows, plan)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.isfinite(o).all()
    off = oracle.q_offsets(inp["q_lens"])
    worst = 0.0
    for b in (0, 1, 31):                      # the 128K request and two 4K ones
        sub = dict(inp, block_table=inp["block_table"][[b]], seq_lens=inp["seq_lens"][[b]],
                   q_lens=inp["q_lens"][[b]], q=inp["q"][off[b]:off[b + 1]])
        ref = ref_prefill(sub)
        worst = max(worst, float(np.abs(o[off[b]:off[b + 1]] - ref).max()))
    print(f"specdec full size: {len(rows)} blocks, sampled max err {worst:.3e}", flush=True)
    assert worst <= TOL["bf16"]


def _rows_ref(inp, b, j0, j1):
    """Oracle output of rows [j0, j1) of request b: a request of its own whose
    cache ends at the last of those rows (same block-table row)."""
    off = oracle.q_offsets(inp["q_lens"])
    n, L = int(inp["q_lens"][b]), int(inp["seq_lens"][b])
    sub = dict(inp, block_table=inp["block_table"][[b]],
               seq_lens=np.array([L - n + j1], np.int32), q_lens=np.array([j1 - j0], np.int32),
               q=inp["q"][off[b] + j0:off[b] + j1])
    return ref_prefill(sub), off[b] + j0


def test_chunked_full_size_sampled():
    """The chunked-prefill workload at full size in the launch configuration
    the benchmark times (default block size and plan): the shortest request
    whole, and the first and last rows of the longest."""
    w = CONFIGS["chunked"]
    inp = make_inputs(w)
    dev = hda.DeviceBatch.from_inputs(inp)
    rows, plan = dev.prefill_plan(inp["q_lens"])
    out = dev.prefill(rows, plan)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.isfinite(o).all()
    kv, ql = inp["seq_lens"], inp["q_lens"]
    short, long_ = int(np.argmin(kv)), int(np.argmax(kv))
    cases = [(short, 0, int(ql[short])), (long_, 0, 3), (long_, int(ql[long_]) - 5, int(ql[long_]))]
    worst = 0.0
    for b, j0, j1 in cases:
        ref, r0 = _rows_ref(inp, b, j0, j1)
        worst = max(worst, float(np.abs(o[r0:r0 + (j1 - j0)] - ref).max()))
    print(f"chunked full size: {len(rows)} blocks of <= {int(rows[:, 2].max())} rows, "
          f"sampled max err {worst:.3e}", flush=True)
    assert worst <= TOL["bf16"]

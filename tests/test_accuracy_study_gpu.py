"""Accuracy of the cache precisions and product modes, measured on the GPU.

One set of float32 draws (long-tail lengths 256..8192, per-kv-head
magnitudes U(0.5, 2)) is stored as a bf16 cache and as fp8 E4M3 caches with
per-tensor, per-head and per-page scales; each runs through the library
(bf16 products, and for tensor/head scales also the native-fp8 products).
Every output is compared with the exact attention (float64) over the bf16
cache, i.e. the values before fp8 quantisation.  A second case multiplies
the V values of each request by 2^-U(0, 24), a magnitude spread wider than
E4M3's range, so that under a per-tensor (or per-head) scale the quietest
requests fall to subnormals or zero.  Errors are reported per output row
(request, q head), relative to that row's rms: median and max over rows,
and the overall relative rms.  The tables are printed (run with -s); the
assertions are sanity bars only: every fp8 variant is farther from the
reference than the bf16 cache; without the spread, finer scales never lose
more than 10% (median row error); with it, page scales keep the worst row
under a quarter of what tensor scales give; native-fp8 products stay within 4x the
error of bf16 products on the same cache.
"""

import numpy as np
import pytest
import torch

import load_balanced_split_step_amd.hda as hda
import oracle
from load_balanced_split_step_amd.workloads import Workload, make_inputs
from tests.gpu_util import need_gpu, scale_kw

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


BASE = Workload("study", 16, 64, 8, 128, 64, len_range=(256, 8192), head_scale=True, seed=90)
SPREAD = BASE.with_(name="study_spread", v_req_spread=24.0)


def _run(inp, math):
    dev = hda.DeviceBatch.from_inputs(inp, math=math)
    lens = inp["seq_lens"]
    out = dev.decode(hda.hda_plan(lens, *hda.launch_config(lens, inp["workload"].n_kv_heads)))
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("base", [BASE, SPREAD], ids=["plain", "v_req_spread_24"])
def test_accuracy_study(base):
    ref_inp = make_inputs(base, poison=False)
    ref = oracle.attention_reference(oracle.bf16_to_f64(ref_inp["q"]), ref_inp["k_pages"],
                                     ref_inp["v_pages"], ref_inp["block_table"],
                                     ref_inp["seq_lens"], "bf16", float(ref_inp["sm_scale"]))
    row_rms = np.sqrt((ref * ref).mean(axis=-1))              # [B, Hq]
    rows = []

    def record(name, out):
        e = out - ref
        rel = np.sqrt((e * e).mean(axis=-1)) / row_rms           # per (request, q head)
        overall = float(np.sqrt((e * e).sum() / (ref * ref).sum()))
        rows.append((name, float(np.median(rel)), float(rel.max()), overall))
        return rows[-1][1], rows[-1][2]

    rms = {"bf16": record("bf16 cache, bf16 products", _run(ref_inp, "bf16"))}
    for mode in ("tensor", "head", "page"):
        inp = make_inputs(base.with_(kv_dtype="fp8", kv_scale=mode), poison=False)
        assert np.array_equal(inp["q"], ref_inp["q"])
        rms[mode] = record(f"fp8 cache, {mode} scales, bf16 products", _run(inp, "bf16"))
        if mode != "page":
            rms[mode + "_n"] = record(f"fp8 cache, {mode} scales, native fp8 products",
                                      _run(inp, "fp8"))
            # the part of it that the q quantisation explains (oracle, exact)
            qe = oracle.attention_fp8q(inp["q"], inp["k_pages"], inp["v_pages"],
                                       inp["block_table"], inp["seq_lens"], "fp8",
                                       float(inp["sm_scale"]), **scale_kw(inp))
            record(f"  (oracle: fp8 cache, {mode} scales, fp8 q, exact weights)", qe)
    print(f"\n{base.name}:\n| variant | median row rel err | max row rel err | overall rel rms "
          f"|\n|---|---|---|---|")
    for name, med, mx, ov in rows:
        print(f"| {name} | {med:.3e} | {mx:.3e} | {ov:.3e} |")
    print("(row rel err = rms of the error over D / rms of the reference row; reference: exact "
          "attention over the bf16 cache)", flush=True)
    med = {k: v[0] for k, v in rms.items()}
    mx = {k: v[1] for k, v in rms.items()}
    assert all(med[m] > med["bf16"] for m in ("tensor", "head", "page"))
    if base.v_req_spread == 0:
        assert med["head"] <= 1.1 * med["tensor"] and med["page"] <= 1.1 * med["head"]
    else:
        assert mx["page"] < 0.25 * mx["tensor"]
    assert med["tensor_n"] <= 4 * med["tensor"] and med["head_n"] <= 4 * med["head"]

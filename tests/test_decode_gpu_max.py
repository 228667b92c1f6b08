"""Parity at a size past the workloads': one long request beside three
short ones (64 q / 8 kv heads, head dim 128, page 64, random page
placement) -- 1,048,576 + 123 cached tokens over a bf16 cache, 2,097,152 +
123 over an fp8 one.  Each K or V pool then spans more than 2 GiB, so the
slabs of its highest-numbered pages sit past byte offset 2^31, and the long
request, which holds nearly every page, reads hundreds of them (the tile
kernel's per-chunk buffer resources start from 64-bit page offsets); the
planner cuts the long request into thousands of tiles.  Through the call
path bench.py times
(hda.launch_config, plan in the launch arguments or stored by
hda_plan_upload, merge of split requests), every output element against the
fp64 oracle; the device check words stay clear.  The same caches with
several query rows per request (multi-token queries: 40 rows on the long
cache, the row blocks and launch shape of the default sizing, the
LDS-shared block kernels and the row merge), every output element against
the oracle as well."""

import pytest
import torch

import load_balanced_split_step_amd.hda as hda
from load_balanced_split_step_amd.workloads import Workload, make_inputs
import oracle
from tests.gpu_util import TOL, max_err, need_gpu, oracle_out, scale_kw

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


LONG = {"bf16": 1048576 + 123, "fp8": 2097152 + 123}    # pool past 2 GiB per dtype


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_million_token_request_every_element(kv):
    lens_in = [LONG[kv], 3000, 70000, 17]
    w = Workload(f"max_{kv}", len(lens_in), 64, 8, 128, 64, kv_dtype=kv, seed=97)
    inp = make_inputs(w, lengths=lens_in)
    lens = inp["seq_lens"]
    n_pages = int(inp["k_pages"].shape[0])
    page_bytes = inp["k_pages"][0].nbytes
    assert n_pages * page_bytes > 2 ** 31, "the pool must extend past 2 GiB"
    dev = hda.DeviceBatch.from_inputs(inp)
    tl, W = hda.launch_config(lens, w.n_kv_heads)
    plan = hda.hda_plan(lens, tl, W)
    print(f"{kv}: {int(lens.sum())} tokens, pool {n_pages * page_bytes / 2**30:.2f} GiB per K/V, "
          f"tile_len {tl}, W {W}, {int(plan[4])} tiles, P {int(plan[6])}, plan {plan.size} ints",
          flush=True)
    out = dev.decode(plan, upload="bench")
    torch.cuda.synchronize()
    assert dev.check(plan) == 0
    ref = oracle_out(inp)
    err = max_err(out, ref)
    print(f"{kv}: {out.numel()} outputs, max |gpu - oracle| {err:.3e}", flush=True)
    assert err <= TOL[kv]


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_million_token_cache_query_rows_every_element(kv):
    q_lens = [40, 5, 33, 1]
    lens_in = [LONG[kv] + q_lens[0], 3000 + q_lens[1], 70000 + q_lens[2], 17 + q_lens[3]]
    w = Workload(f"max_pf_{kv}", len(lens_in), 64, 8, 128, 64, kv_dtype=kv, seed=98)
    inp = make_inputs(w, lengths=lens_in, q_lens=q_lens)
    n_pages = int(inp["k_pages"].shape[0])
    assert n_pages * inp["k_pages"][0].nbytes > 2 ** 31, "the pool must extend past 2 GiB"
    dev = hda.DeviceBatch.from_inputs(inp)
    rows, plan = dev.prefill_plan(inp["q_lens"])
    print(f"{kv}: {len(rows)} row blocks of <= {int(rows[:, 2].max())} rows, "
          f"{int(plan[4])} tiles, P {int(plan[6])}", flush=True)
    out = dev.prefill(rows, plan)
    torch.cuda.synchronize()
    ref = oracle.prefill_reference(oracle.bf16_to_f64(inp["q"]), inp["k_pages"], inp["v_pages"],
                                   inp["block_table"], inp["seq_lens"], inp["q_lens"],
                                   inp["kv_dtype"], float(inp["sm_scale"]), **scale_kw(inp))
    err = max_err(out, ref)
    print(f"{kv}: {out.numel()} outputs, max |gpu - oracle| {err:.3e}", flush=True)
    assert err <= TOL[kv]

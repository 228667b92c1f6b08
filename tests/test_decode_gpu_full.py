"""Full-size parity: every workload at its real size, in the launch
configuration and through the call path bench.py times (hda.launch_config;
the plan in the tile kernel's launch arguments when it fits, else stored by
hda_plan_upload; the merge of split requests), with every output element
checked against the fp64 oracle.  Bar: 2e-2 (bf16 cache) / 6e-2 (fp8 cache)
max-abs error.  The device check words must stay clear (the plan matches the
device lengths)."""

import numpy as np
import pytest
import torch

import load_balanced_split_step_amd.hda as hda
from load_balanced_split_step_amd.workloads import CONFIGS, make_inputs
from tests.gpu_util import TOL, max_err, need_gpu, oracle_out

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


FULL = ["tiny", "uniform", "extreme", "longtail", "fp8", "fp8_page"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_every_element(name):
    w = CONFIGS[name]
    inp = make_inputs(w)
    lens = inp["seq_lens"]
    dev = hda.DeviceBatch.from_inputs(inp)
    tl, W = hda.launch_config(lens, w.n_kv_heads)
    plan = hda.hda_plan(lens, tl, W)
    path = "launch arguments" if plan.size <= hda.HDA_PLAN_ARG_INTS else "hda_plan_upload"
    print(f"{name}: B={len(lens)} tokens={int(lens.sum())} tile_len={tl} W={W} "
          f"P={int(plan[6])} plan {plan.size} ints ({path})", flush=True)
    out = dev.decode(plan, upload="bench")
    torch.cuda.synchronize()
    assert dev.check(plan) == 0
    ref = oracle_out(inp)
    err = max_err(out, ref)
    print(f"{name}: {out.numel()} outputs, max |gpu - oracle| {err:.3e}", flush=True)
    assert err <= TOL[w.kv_dtype]
    if name == "extreme":
        # the static-split baseline at full size reaches the same outputs
        outs = dev.decode(hda.hda_plan_static(lens, 16))
        torch.cuda.synchronize()
        assert max_err(outs, ref) <= TOL["bf16"]

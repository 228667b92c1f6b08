"""hda_decode_noalloc -- hda_decode with its workspace in the library's own
device array, for callers that cannot allocate -- against hda_decode with a
caller workspace, through the C ABI: bitwise-equal outputs on two calls in a
row, the second with a smaller batch (the plan in the launch arguments,
then in device memory; bf16, then fp8 with the prologue, whose q' also lives
in the workspace), each also within the fp64 oracle's bar; a plan whose
workspace exceeds HDA_NOALLOC_WORKSPACE_BYTES is refused before any launch.
"""

import ctypes

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


def _vp(x):
    return ctypes.c_void_p(x.data_ptr()) if x is not None else None


def _decode(lib_fn, dev, plan, plan_dev, out):
    p = dev.params(plan)                     # a caller workspace (ignored by noalloc)
    t = dev.t
    plan = np.ascontiguousarray(plan, dtype=np.int32)
    st = lib_fn(ctypes.byref(p), _vp(t["q"]), _vp(t["k_pages"]), _vp(t["v_pages"]),
                _vp(t["block_table"]), _vp(t["seq_lens"]), hda._i32p(plan), _vp(plan_dev),
                plan.size, _vp(out), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


def _compare(w, lens, plan_in_args):
    lib = hda.load_library()
    inp = make_inputs(w, lengths=lens)
    L = inp["seq_lens"]
    plan = hda.hda_plan(L, *hda.launch_config(L, w.n_kv_heads))
    assert plan.size <= hda.HDA_PLAN_ARG_INTS
    need = hda.hda_workspace_bytes(plan, w.n_q_heads, w.n_kv_heads, w.head_dim)
    assert 0 < need <= hda.HDA_NOALLOC_WORKSPACE_BYTES
    pd = None if plan_in_args else torch.from_numpy(plan).cuda()
    shape = (len(L), w.n_q_heads, w.head_dim)
    ref_out = torch.full(shape, float("nan"), device="cuda:0")
    out = torch.full(shape, float("nan"), device="cuda:0")
    dev = hda.DeviceBatch.from_inputs(inp)
    assert _decode(lib.hda_decode, dev, plan, pd, ref_out) == hda.HDA_OK
    dev2 = hda.DeviceBatch.from_inputs(inp)      # fresh cache copy (the prologue writes it)
    assert _decode(lib.hda_decode_noalloc, dev2, plan, pd, out) == hda.HDA_OK
    torch.cuda.synchronize()
    print(f"{w.name}: B={len(L)} P={int(plan[6])} workspace {need} bytes, "
          f"plan {'in launch arguments' if plan_in_args else 'in device memory'}", flush=True)
    assert torch.equal(out, ref_out)
    assert torch.equal(dev.t["k_pages"], dev2.t["k_pages"])
    assert max_err(out, oracle_out(inp)) <= TOL[w.kv_dtype]


def test_noalloc_matches_decode_two_calls_second_smaller():
    big = CONFIGS["longtail"].with_(name="na_big", batch=24, len_range=(64, 20000))
    small = CONFIGS["extreme"].with_(name="na_small", batch=5)
    _compare(big, None, plan_in_args=True)
    _compare(small, [9000, 700, 17, 1, 2048], plan_in_args=False)


def test_noalloc_with_prologue_two_calls_second_smaller():
    _compare(CONFIGS["fp8"].with_(name="na_fp8", batch=40, len_range=(64, 6000)), None, True)
    _compare(CONFIGS["fp8"].with_(name="na_fp8s", batch=3, len_range=(64, 6000)), None, False)


def test_noalloc_refuses_a_plan_beyond_its_workspace():
    lib = hda.load_library()
    B, Hq, Hkv, D = 128, 64, 8, 128
    lens = np.full(B, 8192, np.int32)
    plan = hda.hda_plan(lens, 16, 1024)
    assert hda.hda_workspace_bytes(plan, Hq, Hkv, D) > hda.HDA_NOALLOC_WORKSPACE_BYTES
    # small real buffers: nothing is launched, so nothing is read
    t = torch.zeros(1 << 16, dtype=torch.int32, device="cuda:0")
    p = hda.hda_params(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, page_size=64,
                       max_pages_per_req=128, num_pages=B * 128, kv_dtype=hda.HDA_KV_BF16,
                       sm_scale=D ** -0.5, k_scale=1.0, v_scale=1.0)
    vp = ctypes.c_void_p(t.data_ptr())
    st = lib.hda_decode_noalloc(ctypes.byref(p), vp, vp, vp, vp, vp, hda._i32p(plan), vp,
                                plan.size, vp, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == hda.HDA_ERR_WORKSPACE

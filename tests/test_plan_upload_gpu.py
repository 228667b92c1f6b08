"""The plan upload through store-kernel launch arguments (hda_plan_upload):
every int arrives exactly, in one launch or several, nothing past the plan is
written, the host buffer may be reused as soon as the call returns, and a
decode step with an uploaded plan is bitwise the step with a copied plan."""

import numpy as np
import pytest
import torch

import load_balanced_split_step_amd.hda as hda
from load_balanced_split_step_amd.workloads import CONFIGS, make_inputs
from tests.gpu_util import need_gpu

pytestmark = pytest.mark.gpu

SENTINEL = -123456789


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


@pytest.mark.parametrize("n", [1, 7, 255, 256, 257, 999, 1000, 1001, 1999, 2000, 2001, 5003])
def test_upload_exact(n):
    rng = np.random.default_rng(n)
    plan = rng.integers(-2**31, 2**31, size=n, dtype=np.int64).astype(np.int32)
    dst = torch.full((n + 64,), SENTINEL, dtype=torch.int32, device="cuda:0")
    hda.hda_plan_upload(plan, dst)
    torch.cuda.synchronize()
    got = dst.cpu().numpy()
    assert np.array_equal(got[:n], plan)
    assert (got[n:] == SENTINEL).all()


def test_upload_host_buffer_reusable():
    n = 2345
    host = np.arange(n, dtype=np.int32)
    want = [host.copy()]
    dsts = [torch.full((n,), SENTINEL, dtype=torch.int32, device="cuda:0") for _ in range(6)]
    if hasattr(torch.cuda, "_sleep"):
        torch.cuda._sleep(2_000_000)       # keep the stream busy while the host rewrites
    for j, d in enumerate(dsts):
        hda.hda_plan_upload(host, d)
        host[:] = host * 3 + j + 1         # overwritten right after the call returns
        want.append(host.copy())
    torch.cuda.synchronize()
    for j, d in enumerate(dsts):
        assert np.array_equal(d.cpu().numpy(), want[j]), j


@pytest.mark.parametrize("cfg,tile_len,W", [("tiny", 64, 8), ("uniform", 128, 64),
                                            ("extreme", 128, 64), ("extreme", 128, 63)])
def test_decode_with_uploaded_plan_bitwise(cfg, tile_len, W):
    inp = make_inputs(CONFIGS[cfg])
    dev = hda.DeviceBatch.from_inputs(inp, device="cuda:0")
    plan = hda.hda_plan(inp["seq_lens"], tile_len, W)
    copied = torch.from_numpy(plan).cuda()
    uploaded = torch.full((plan.size,), SENTINEL, dtype=torch.int32, device="cuda:0")
    hda.hda_plan_upload(plan, uploaded)
    a = dev.decode(plan, plan_dev=copied)
    b = dev.decode(plan, plan_dev=uploaded)
    torch.cuda.synchronize()
    assert np.array_equal(uploaded.cpu().numpy(), plan)
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    if plan.size <= hda.HDA_PLAN_ARG_INTS:
        # the plan in the tile kernel's launch arguments (the bench's path)
        c = _decode_plan_in_args(dev, plan)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int32), c.view(torch.int32))
    print(f"{cfg}: {plan.size} plan ints, outputs bitwise equal", flush=True)


def _decode_plan_in_args(dev, plan):
    """hda_decode with no device copy of the plan: it rides in the launch."""
    t = dev.t
    out = torch.empty((dev.kw["batch"], dev.kw["n_q_heads"], dev.kw["head_dim"]),
                      dtype=torch.float32, device=dev.device)
    hda.hda_decode(dev.params(plan), t["q"], t["k_pages"], t["v_pages"], t["block_table"],
                   t["seq_lens"], plan, None, out)
    return out


ARG_CASES = ["tiny", "extreme_s", "longtail_s", "fp8_s", "fp8_page_s", "fp8_head_s", "tiny_page"]


@pytest.mark.parametrize("name", ARG_CASES + ["fp8_s/native"])
def test_decode_plan_in_launch_arguments(name):
    """Every kernel variant (D 64 and 128, bf16 and fp8 caches, tensor, head
    and page scales, native-fp8 products): outputs bitwise those of the same
    plan read from device memory, and within the oracle bar."""
    from tests.test_decode_gpu import SCALED, plans_for
    from tests.gpu_util import TOL, oracle_out, max_err
    cfg, _, math = name.partition("/")
    w, lens = SCALED[cfg]
    inp = make_inputs(w, lengths=lens)
    ref = oracle_out(inp)
    dev = hda.DeviceBatch.from_inputs(inp, math=math or "bf16")
    n = 0
    for pname, plan in plans_for(inp["seq_lens"], w.n_kv_heads):
        if plan.size > hda.HDA_PLAN_ARG_INTS:
            continue
        a = _decode_plan_in_args(dev, plan)
        b = dev.decode(plan)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), (name, pname)
        err = max_err(a, ref)
        assert err <= TOL[w.kv_dtype], (name, pname, err)
        n += 1
    print(f"{name}: {n} plans in launch arguments, bitwise equal", flush=True)
    assert n >= 3


def _lengths_for_plan_size(size):
    """Seeded search for a batch whose plan has exactly `size` ints."""
    rng = np.random.default_rng(5)
    while True:
        B, W, tl = int(rng.integers(30, 140)), int(rng.integers(8, 300)), int(rng.choice([64, 128]))
        lens = rng.integers(1, 1500, size=B).astype(np.int32)
        if hda.hda_plan_capacity(B, W) < size:
            continue
        plan = hda.hda_plan(lens, tl, W)
        if plan.size == size:
            return lens, plan


def test_plan_in_launch_arguments_at_the_limit():
    """The longest plan the launch arguments take (HDA_PLAN_ARG_INTS ints)
    gives the device-plan outputs bitwise; one int more is refused."""
    lens, plan = _lengths_for_plan_size(hda.HDA_PLAN_ARG_INTS)
    w = CONFIGS["tiny"].with_(name="arg_limit", batch=len(lens))
    inp = make_inputs(w, lengths=lens)
    dev = hda.DeviceBatch.from_inputs(inp)
    a = _decode_plan_in_args(dev, plan)
    b = dev.decode(plan)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    lens2, plan2 = _lengths_for_plan_size(hda.HDA_PLAN_ARG_INTS + 1)
    inp2 = make_inputs(CONFIGS["tiny"].with_(name="arg_over", batch=len(lens2)), lengths=lens2)
    dev2 = hda.DeviceBatch.from_inputs(inp2)
    with pytest.raises(hda.HdaError) as e:
        _decode_plan_in_args(dev2, plan2)
    assert e.value.status == hda.HDA_ERR_UNSUPPORTED
    print(f"{plan.size} ints in the launch arguments; {plan2.size} refused", flush=True)

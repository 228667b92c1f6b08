"""Full-size parity: each workload at its real size, in the launch
configuration bench.py times (hda.launch_config), checked on sampled
(request, q head) outputs that the fp64 oracle computes one by one, plus a
property that holds for every output at any size: each output dim lies
within the range of that request's V values (softmax weights form a convex
combination).  Bar: 2e-2 (bf16 cache) / 6e-2 (fp8 cache) max-abs error."""

import numpy as np
import pytest
import torch

import load_balanced_split_step_amd.hda as hda
import oracle
from load_balanced_split_step_amd.workloads import CONFIGS, make_inputs
from tests.gpu_util import TOL, need_gpu, oracle_inputs, scale_kw

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def sample_pairs(lens, n_q_heads, group, seed):
    rng = np.random.default_rng(seed)
    B = len(lens)
    bs = {int(np.argmax(lens)), int(np.argmin(lens)), 0, B - 1}
    bs |= set(rng.choice(B, size=min(B, 4), replace=False).tolist())
    pairs = []
    for b in sorted(bs):
        for h in {0, n_q_heads - 1, group - 1, int(rng.integers(n_q_heads))}:
            pairs.append((b, h))
    return pairs


def v_range_check(out, inp, vpool, n_req=None):
    """min_t V <= out <= max_t V per (request, q head, dim), on the cache the
    oracle attends (values decoded exactly)."""
    w = inp["workload"]
    g = w.group
    ps = w.page_size
    o = out.cpu().numpy()
    B = len(inp["seq_lens"])
    kw = scale_kw(inp)
    for b in range(B if n_req is None else min(B, n_req)):
        L = int(inp["seq_lens"][b])
        vs = oracle.row_scales(kw["v_scale"], kw["scale_mode"], kw["v_scales"],
                               inp["block_table"][b], L, ps, w.n_kv_heads)   # [L, Hkv]
        v = oracle.decode_kv(oracle.gather_request(vpool, inp["block_table"][b], L, ps),
                             w.kv_dtype, vs[:, :, None])                      # [L, Hkv, D]
        lo, hi = v.min(axis=0), v.max(axis=0)                               # [Hkv, D]
        for h in range(w.n_q_heads):
            kvh = h // g
            slack = 1e-3 * max(1.0, float(np.abs(v[:, kvh]).max()))
            assert np.all(o[b, h] >= lo[kvh] - slack) and np.all(o[b, h] <= hi[kvh] + slack), (b, h)


@pytest.mark.parametrize("name", ["uniform", "extreme", "longtail", "fp8", "fp8_page"])
def test_full_size_sampled(name):
    w = CONFIGS[name]
    inp = make_inputs(w)
    lens = inp["seq_lens"]
    print(f"{name}: B={len(lens)} tokens={int(lens.sum())}", flush=True)
    dev = hda.DeviceBatch.from_inputs(inp)
    tl, W = hda.launch_config(lens, w.n_kv_heads)
    out = dev.decode(hda.hda_plan(lens, tl, W))
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    q, kp, vp, _ = oracle_inputs(inp)
    pairs = sample_pairs(lens, w.n_q_heads, w.group, seed=w.seed)
    ref = oracle.attention_selected(q, kp, vp, inp["block_table"], lens, w.kv_dtype,
                                    float(inp["sm_scale"]), pairs, **scale_kw(inp))
    o = out.cpu().numpy()
    err = max(float(np.abs(o[b, h] - ref[(b, h)]).max()) for b, h in pairs)
    print(f"{name}: {len(pairs)} sampled (b, h), max err {err:.3e}", flush=True)
    assert err <= TOL[w.kv_dtype]
    v_range_check(out, inp, vp, n_req=8)
    if name == "extreme":
        # the static-split baseline at full size reaches the same outputs
        outs = dev.decode(hda.hda_plan_static(lens, 16))
        torch.cuda.synchronize()
        assert float((outs - out).abs().max()) <= TOL["bf16"]

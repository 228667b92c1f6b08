"""GPU parity of the native-fp8 product mode (math "fp8": QK^T and PV on fp8
MFMA operands, V pages dim-major).

The q quantisation is deterministic and the oracle replays it exactly
(attention_fp8q); the fp8 rounding of the softmax weights is bounded from
the exact weights (weight_rounding_bounds), with the accumulation error of
the matrix cores' fp8 products (about 2^-14 of the summed magnitudes,
measured; 2^-12 assumed) in the scores and the token sums.  Bar, per output
element: |gpu - oracle| <= that worst-case bound + 1e-6 (float32 epilogue
and merge); and over all elements of a run the squared error stays within
4x the expected squared error.  The distance to the exact attention with an unquantised q
(the plain definition over the fp8 cache, fp64) is held to the fp8-cache
bar, 6e-2 max-abs, like every other mode: at the scaled sizes here and, for
every output element, at the full size of the fp8 workload through the call
path bench.py times.  Also: device-planned launches bitwise equal
to host-planned ones, and the prologue's column write into dim-major V
pages (attention after it within the fp8 bar of the fp64 oracle with the
bf16 q', the q quantisation included in that bar's slack).
"""

import numpy as np
import pytest
import torch

import load_balanced_split_step_amd.hda as hda
import oracle
from load_balanced_split_step_amd.workloads import CONFIGS, Workload, make_inputs
from tests.gpu_util import TOL, need_gpu, oracle_inputs, scale_kw, max_err

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


CASES = {
    "fp8n_s": (CONFIGS["fp8"].with_(name="fp8n_s", batch=12, len_range=(30, 3000), prologue=False),
               None),
    "fp8n_head": (CONFIGS["fp8"].with_(name="fp8n_head", batch=8, len_range=(1, 2500),
                                       prologue=False, kv_scale="head", head_scale=True), None),
    "fp8n_page128": (Workload("fp8n_page128", 6, 32, 4, 128, 128, kv_dtype="fp8", seed=71),
                     [1, 64, 65, 127, 128, 1500]),
    "fp8n_group16": (Workload("fp8n_group16", 5, 32, 2, 128, 64, kv_dtype="fp8", seed=72),
                     [300, 64, 5, 2000, 129]),
}


def plans_for(lens, n_kv_heads):
    tl, W = hda.launch_config(lens, n_kv_heads)
    out = [("dyn-default", hda.hda_plan(lens, tl, W))]
    for tl2, W2 in [(64, 7), (100, 13), (32, 200), (512, 3)]:
        out.append((f"dyn-{tl2}-{W2}", hda.hda_plan(lens, tl2, W2)))
    for S in (1, 3):
        out.append((f"static-{S}", hda.hda_plan_static(lens, S)))
    return out


def all_pairs(inp):
    return [(b, h) for b in range(len(inp["seq_lens"])) for h in range(inp["workload"].n_q_heads)]


# Accumulation error of the fp8 matrix-core products, relative to the sum of
# the magnitudes they add (a probe measured about 2^-14; 4x margin): the
# scores' error and the token sums' error in the bound.
MFMA_EPS = 2.0 ** -12


def check_against_bounds(out, inp, q_raw, pairs, label):
    q_eff = oracle.dequantized_q(q_raw)
    kw = scale_kw(inp)
    res = oracle.weight_rounding_bounds(q_eff, inp["k_pages"], inp["v_pages"], inp["block_table"],
                                        inp["seq_lens"], "fp8", float(inp["sm_scale"]), pairs,
                                        score_eps=MFMA_EPS, sum_eps=MFMA_EPS, **kw)
    o = out.detach().cpu().numpy().astype(np.float64)
    assert np.isfinite(o).all()
    err2 = pred2 = 0.0
    worst_ratio = 0.0
    for (b, h) in pairs:
        ref, worst, rms = res[(b, h)]
        e = np.abs(o[b, h] - ref)
        assert np.all(e <= worst + 1e-6), (label, b, h, float(e.max()), float(worst.min()))
        worst_ratio = max(worst_ratio, float((e / (worst + 1e-6)).max()))
        err2 += float((e * e).sum())
        pred2 += float((rms * rms).sum())
    print(f"{label}: max err/bound {worst_ratio:.3f}, rms err / expected "
          f"{np.sqrt(err2 / max(pred2, 1e-300)):.3f}", flush=True)
    assert err2 <= 4.0 * pred2 + len(pairs) * 128 * 1e-10, (label, err2, pred2)


@pytest.mark.parametrize("name", list(CASES))
def test_parity_native_fp8(name):
    w, lens = CASES[name]
    inp = make_inputs(w, lengths=lens)
    dev = hda.DeviceBatch.from_inputs(inp, math="fp8")
    exact = oracle.attention_reference(oracle.bf16_to_f64(inp["q"]), inp["k_pages"], inp["v_pages"],
                                       inp["block_table"], inp["seq_lens"], "fp8",
                                       float(inp["sm_scale"]), **scale_kw(inp))
    pairs = all_pairs(inp)
    for pname, plan in plans_for(inp["seq_lens"], w.n_kv_heads):
        out = dev.decode(plan)
        torch.cuda.synchronize()
        check_against_bounds(out, inp, inp["q"], pairs, f"{name} {pname}")
        err = max_err(out, exact)
        print(f"{name} {pname}: max |diff| vs unquantised-q attention {err:.3e}", flush=True)
        assert err <= TOL["fp8"], (name, pname, err)


def test_native_device_plan_bitwise_equals_host_plan():
    w, lens = CASES["fp8n_s"]
    inp = make_inputs(w, lengths=lens)
    dev = hda.DeviceBatch.from_inputs(inp, math="fp8")
    L = inp["seq_lens"]
    for tl, W in [(128, 64), (64, 7), (100, 300)]:
        a = dev.decode(hda.hda_plan(L, tl, W))
        b = dev.decode_auto(tl, W)
        torch.cuda.synchronize()
        assert torch.equal(a, b), (tl, W)


def _q_prime_from_workspace(dev, plan, B, Hq, D):
    """The prologue's q' (bf16 bits [B, Hq, D]) from the workspace, at the
    offset the header documents: after the check words int32 [W][Hkv], the
    partial outputs float32 [P][Hq][D] and partial log-sum-exps float32
    [P][Hq], each region 256-aligned."""
    r256 = lambda x: (x + 255) // 256 * 256
    W, P = int(plan[3]), int(plan[6])
    off = r256(W * dev.kw["n_kv_heads"] * 4) + r256(P * Hq * D * 4) + r256(P * Hq * 4)
    raw = dev._ws[off:off + B * Hq * D * 2].cpu().numpy()
    return raw.view(np.uint16).reshape(B, Hq, D)


def test_native_prologue_writes_dim_major_column():
    w = CONFIGS["fp8"].with_(name="fp8n_pro", batch=9, len_range=(16, 1500))
    inp = make_inputs(w)
    q_p, kp, vp, (kc, vc, kx, vx) = oracle_inputs(inp)
    dev = hda.DeviceBatch.from_inputs(inp, math="fp8")
    plan = hda.hda_plan(inp["seq_lens"], 128, 11)
    out = dev.decode(plan)
    torch.cuda.synchronize()
    shape = inp["v_pages"].shape
    vdev = dev.v_pages_token_major(shape)
    ps = shape[2]
    for b, L in enumerate(inp["seq_lens"].tolist()):
        page = inp["block_table"][b][(L - 1) // ps]
        got, want = vdev[page, :, (L - 1) % ps, :], vc[b]
        diff = got != want
        if diff.any():   # another code only where the value is within float32 error of a midpoint
            mid = (oracle.fp8_decode(got[diff]) + oracle.fp8_decode(want[diff])) / 2
            assert np.all(np.abs(vx[b][diff] - mid) <= 1e-5 * np.maximum(1.0, np.abs(vx[b][diff])))
    # every other V element is unchanged
    mask = np.ones((shape[0], ps), dtype=bool)
    for b, L in enumerate(inp["seq_lens"].tolist()):
        mask[inp["block_table"][b][(L - 1) // ps], (L - 1) % ps] = False
    before = inp["v_pages"].transpose(0, 2, 1, 3)[mask]
    after = vdev.transpose(0, 2, 1, 3)[mask]
    assert np.array_equal(before, after)
    # q' as the kernel stored it: within one bf16 step of the oracle's q'
    qk = _q_prime_from_workspace(dev, plan, w.batch, w.n_q_heads, w.head_dim)
    qk64 = oracle.bf16_to_f64(qk)
    assert np.all(np.abs(qk64 - q_p) <= 2.0 ** -8 * np.abs(q_p) + 1e-30)
    # attention after the write, from that q': within the fp8 weight-rounding bound
    inp2 = dict(inp, k_pages=kp, v_pages=vp)
    check_against_bounds(out, inp2, qk, all_pairs(inp), "native prologue")


def test_native_full_size_every_element():
    """The fp8 workload at full size (prologue off: the mode's own check of
    the written token is above), bench.py's launch configuration and plan
    path: every output within 6e-2 of the plain fp64 oracle, and within the
    weight-rounding bound on a sample of rows."""
    w = CONFIGS["fp8"].with_(prologue=False)
    inp = make_inputs(w)
    lens = inp["seq_lens"]
    dev = hda.DeviceBatch.from_inputs(inp, math="fp8")
    tl, W = hda.launch_config(lens, w.n_kv_heads)
    plan = hda.hda_plan(lens, tl, W)
    out = dev.decode(plan, upload="bench")
    torch.cuda.synchronize()
    exact = oracle.attention_reference(oracle.bf16_to_f64(inp["q"]), inp["k_pages"], inp["v_pages"],
                                       inp["block_table"], lens, "fp8", float(inp["sm_scale"]),
                                       **scale_kw(inp))
    err = max_err(out, exact)
    print(f"fp8 full size, native: {out.numel()} outputs, max |gpu - oracle| {err:.3e}",
          flush=True)
    assert err <= TOL["fp8"]
    rng = np.random.default_rng(w.seed)
    bs = sorted({int(np.argmax(lens)), int(np.argmin(lens))} |
                set(rng.choice(len(lens), size=6, replace=False).tolist()))
    pairs = [(b, h) for b in bs for h in range(w.n_q_heads)]
    check_against_bounds(out, inp, inp["q"], pairs, "fp8 full size, native")

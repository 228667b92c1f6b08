"""Device-side planning on the GPU: hda_plan_device writes exactly the plan
hda_plan builds on the host, and hda_decode_auto (items derived inside the
tile kernel) gives outputs bitwise identical to hda_decode with the host
plan, also across decode steps with growing lengths."""

import numpy as np
import pytest
import torch

import load_balanced_split_step_amd.hda as hda
from load_balanced_split_step_amd.workloads import CONFIGS, Workload, draw_lengths, make_inputs
from tests.gpu_util import TOL, need_gpu, oracle_out, max_err

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def device_plan(lens, tile_len, W):
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    cap = hda.hda_plan_capacity(len(lens), W)
    d_lens = torch.from_numpy(lens).cuda()
    d_plan = torch.full((cap,), -7, dtype=torch.int32, device="cuda:0")
    hda.hda_plan_device(d_lens, len(lens), tile_len, W, d_plan, cap)
    torch.cuda.synchronize()
    return d_plan.cpu().numpy()


def test_device_plan_matches_host_plan():
    cases = []
    for name, w in CONFIGS.items():
        lens = draw_lengths(w, w.seed)
        for tl in (16, 128, 512):
            for W in (1, 7, 64, 1024):
                cases.append((lens, tl, W))
    rng = np.random.default_rng(3)
    for _ in range(150):
        B = int(rng.integers(1, 300))
        lens = rng.integers(1, int(rng.choice([5, 200, 20000])) + 1, size=B)
        cases.append((lens, int(rng.integers(1, 400)), int(rng.integers(1, 700))))
    for lens, tl, W in cases:
        want = hda.hda_plan(lens, tl, W)
        got = device_plan(lens, tl, W)
        assert np.array_equal(got[:want.size], want), (len(lens), tl, W)
    print(f"{len(cases)} plans bit-exact", flush=True)


AUTO = [
    ("tiny", CONFIGS["tiny"], None, [(64, 8), (16, 1), (1, 97)]),
    ("extreme_s", CONFIGS["extreme"].with_(name="extreme_s", batch=8), [16384] + [1000] * 7,
     [(128, 64), (64, 7), (100, 300)]),
    ("many", Workload("many", 150, 16, 2, 128, 16, seed=61), None, [(32, 64), (16, 500), (256, 3)]),
    ("fp8_s", CONFIGS["fp8"].with_(name="fp8_s", batch=70, len_range=(20, 2000)), None,
     [(128, 64), (64, 13)]),
    ("fp8_page_s", CONFIGS["fp8_page"].with_(name="fp8_page_s", batch=20, len_range=(20, 3000)),
     None, [(128, 64), (32, 100)]),
]


@pytest.mark.parametrize("name,w,lens,plans", AUTO, ids=[a[0] for a in AUTO])
def test_decode_auto_bitwise_equals_host_plan(name, w, lens, plans):
    if lens is None and w.lengths is None and w.len_range is None:
        lens = list(np.random.default_rng(w.seed).integers(1, 900, size=w.batch))
    inp = make_inputs(w, lengths=lens)
    L = inp["seq_lens"]
    ref = oracle_out(inp)
    dev = hda.DeviceBatch.from_inputs(inp)
    for tl, W in plans:
        a = dev.decode(hda.hda_plan(L, tl, W))
        b = dev.decode_auto(tl, W)
        torch.cuda.synchronize()
        assert torch.equal(a, b), (name, tl, W)
        err = max_err(b, ref)
        print(f"{name} auto tl={tl} W={W}: bitwise equal to host plan, max err {err:.3e}", flush=True)
        assert err <= TOL[w.kv_dtype]


def test_decode_auto_growth_steps():
    """Lengths change in device memory between steps; no host planning."""
    import oracle
    from oracle.prologue import prologue_step, write_new_token
    steps = 3
    w = CONFIGS["fp8"].with_(name="grow_auto", batch=5, len_range=(30, 400))
    L0 = make_inputs(w)["seq_lens"].copy()
    inp = make_inputs(w, lengths=L0 + steps)
    dev = hda.DeviceBatch.from_inputs(inp)
    kp_ref, vp_ref = inp["k_pages"].copy(), inp["v_pages"].copy()
    for s in range(steps + 1):
        lens = (L0 + s).astype(np.int32)
        dev.t["seq_lens"].copy_(torch.from_numpy(lens))
        out = dev.decode_auto(64, 11)
        q_p, _, _, kc, vc = prologue_step(inp["q"], inp["k_new"], inp["v_new"], inp["q_norm_w"],
                                          inp["k_norm_w"], lens, float(inp["rms_eps"]),
                                          float(inp["rope_theta"]), "fp8", float(inp["k_scale"]),
                                          float(inp["v_scale"]))
        kp_ref, vp_ref = write_new_token(kp_ref, vp_ref, inp["block_table"], lens, kc, vc)
        ref = oracle.attention_reference(q_p, kp_ref, vp_ref, inp["block_table"], lens, "fp8",
                                         float(inp["sm_scale"]), float(inp["k_scale"]),
                                         float(inp["v_scale"]))
        torch.cuda.synchronize()
        err = max_err(out, ref)
        print(f"auto growth step {s}: max err {err:.3e}", flush=True)
        assert err <= TOL["fp8"]


def test_graph_replay_of_device_planned_step():
    """One device-planned step captured in a HIP graph; each replay, with
    eager work and synchronisation between replays, equals the eager step,
    also after the lengths change in device memory (re-planned on replay)."""
    w = CONFIGS["extreme"].with_(name="graph_s", batch=8)
    lens0 = np.array([9000] + [700] * 7, dtype=np.int32)
    inp = make_inputs(w, lengths=lens0 + 40)            # room to grow
    dev = hda.DeviceBatch.from_inputs(inp)
    tl, W = 128, 24
    out_g = torch.empty((8, 64, 128), dtype=torch.float32, device="cuda:0")
    dev.t["seq_lens"].copy_(torch.from_numpy(lens0))
    p = dev.params_auto(tl, W)
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        hda.hda_decode_auto(p, dev.t["q"], dev.t["k_pages"], dev.t["v_pages"], dev.t["block_table"],
                            dev.t["seq_lens"], tl, W, out_g)
    torch.cuda.synchronize()
    for step, grow in enumerate([0, 0, 5, 17, 40, 3]):
        lens = lens0 + grow
        dev.t["seq_lens"].copy_(torch.from_numpy(lens))
        g.replay()
        torch.cuda.synchronize()
        eager = dev.decode(hda.hda_plan(lens, tl, W))       # eager work between replays
        _ = (eager * 2).sum().item()
        torch.cuda.synchronize()
        assert torch.equal(out_g, eager), step
        print(f"graph replay {step} (lengths +{grow}): equal to eager", flush=True)


@pytest.mark.parametrize("cfg", ["uniform", "fp8"])
def test_decode_auto_empty_slots(cfg):
    """Batch slots left empty between steps (device length 0) get no item:
    their output rows are not written (they keep what the buffer held), the
    prologue writes no new token for them (their pages keep every byte), and
    the other requests equal the oracle over the requests that have tokens."""
    import oracle
    from oracle.prologue import prologue_step, write_new_token
    lens_full = np.array([700, 300, 1500, 90, 2100, 40], dtype=np.int32)
    empty = np.array([False, True, False, True, False, False])
    w = CONFIGS[cfg].with_(name=f"empty_{cfg}", batch=6, lengths=None, len_range=None)
    inp = make_inputs(w, lengths=lens_full)
    dev = hda.DeviceBatch.from_inputs(inp)
    lens = np.where(empty, 0, lens_full).astype(np.int32)
    dev.t["seq_lens"].copy_(torch.from_numpy(lens))
    ps = int(inp["k_pages"].shape[2])
    k_before = dev.t["k_pages"].clone()
    v_before = dev.t["v_pages"].clone()
    sentinel = 12345.0
    out = torch.full((6, w.n_q_heads, w.head_dim), sentinel, dtype=torch.float32, device="cuda:0")
    dev.decode_auto(64, 9, out=out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(got[empty] == sentinel)
    sel = ~empty
    bt = inp["block_table"][sel]
    kp, vp = inp["k_pages"], inp["v_pages"]
    if w.prologue:
        q_p, _, _, kc, vc = prologue_step(inp["q"][sel], inp["k_new"][sel], inp["v_new"][sel],
                                          inp["q_norm_w"], inp["k_norm_w"], lens[sel],
                                          float(inp["rms_eps"]), float(inp["rope_theta"]),
                                          w.kv_dtype, float(inp["k_scale"]), float(inp["v_scale"]))
        kp, vp = write_new_token(kp, vp, bt, lens[sel], kc, vc)
    else:
        q_p = oracle.bf16_to_f64(inp["q"][sel])
    ref = oracle.attention_reference(q_p, kp, vp, bt, lens[sel], w.kv_dtype,
                                     float(inp["sm_scale"]), float(inp["k_scale"]),
                                     float(inp["v_scale"]))
    err = float(np.abs(got[sel] - ref).max())
    print(f"{cfg}: empty slots untouched, others max err {err:.3e}", flush=True)
    assert err <= TOL[w.kv_dtype]
    # the empty requests' pages hold the bytes they held before the step
    page_bytes = k_before.numel() // int(inp["k_pages"].shape[0])
    for b in np.flatnonzero(empty):
        for pg in inp["block_table"][b][:(int(lens_full[b]) + ps - 1) // ps]:
            s = slice(int(pg) * page_bytes, (int(pg) + 1) * page_bytes)
            assert torch.equal(dev.t["k_pages"][s], k_before[s]), (b, int(pg))
            assert torch.equal(dev.t["v_pages"][s], v_before[s]), (b, int(pg))

"""Structure of the seeded synthetic workloads (CPU only)."""

import numpy as np
import pytest

from load_balanced_split_step_amd.workloads import CONFIGS, Workload, make_inputs, draw_lengths, kv_bytes


def test_lengths_follow_recipe():
    assert draw_lengths(CONFIGS["extreme"], 2).tolist() == [131072] + [4096] * 31
    lt = draw_lengths(CONFIGS["longtail"], 3)
    assert len(lt) == 64 and lt.min() >= 256 and lt.max() <= 65536
    f8 = draw_lengths(CONFIGS["fp8"], 4)
    assert len(f8) == 128 and f8.min() >= 1024 and f8.max() <= 32768
    assert np.array_equal(draw_lengths(CONFIGS["longtail"], 3), lt)      # seeded


def test_inputs_deterministic_and_well_formed():
    w = Workload("t", 6, 8, 2, 32, 16, seed=9, head_scale=True)
    lens = [1, 15, 16, 17, 100, 64]
    a = make_inputs(w, lengths=lens)
    b = make_inputs(w, lengths=lens)
    for k in ("q", "k_pages", "v_pages", "block_table"):
        assert np.array_equal(a[k], b[k])
    bt = a["block_table"]
    used = bt[bt >= 0]
    assert sorted(used.tolist()) == list(range(a["k_pages"].shape[0]))   # every page once
    for i, L in enumerate(lens):
        n = -(-L // 16)
        assert (bt[i, :n] >= 0).all() and (bt[i, n:] == -1).all()
        last = bt[i, n - 1]
        # rows past len in the last page are NaN-poisoned, earlier rows finite
        tail = a["k_pages"][last, :, L - (n - 1) * 16:, :]
        assert (tail == 0x7FC0).all()
        assert not (a["k_pages"][last, :, :L - (n - 1) * 16, :] == 0x7FC0).any()


def test_prologue_slot_poisoned_and_scales():
    w = Workload("p", 3, 8, 2, 32, 16, kv_dtype="fp8", prologue=True, seed=4)
    a = make_inputs(w, lengths=[5, 16, 33])
    for i, L in enumerate([5, 16, 33]):
        pg = a["block_table"][i, (L - 1) // 16]
        assert (a["k_pages"][pg, :, (L - 1) % 16, :] == 0x7F).all()
    assert a["k_scale"] > 0 and a["v_scale"] > 0
    assert a["k_new"].shape == (3, 2, 32) and a["q_norm_w"].shape == (32,)


def test_kv_bytes_extreme():
    w = CONFIGS["extreme"]
    inp = {"workload": w, "seq_lens": np.array(w.lengths)}
    assert kv_bytes(inp) == 258048 * 8 * 128 * 2 * 2


@pytest.mark.parametrize("mode", ["tensor", "head", "page"])
def test_fp8_scale_granularity(mode):
    from oracle.codec import fp8_decode
    w = CONFIGS["tiny"].with_(kv_dtype="fp8", kv_scale=mode, head_scale=True, placement="random")
    a = make_inputs(w, poison=False)
    assert a["scale_mode"] == mode
    for pool, sc in ((a["k_pages"], a["k_scales"]), (a["v_pages"], a["v_scales"])):
        mag = np.abs(fp8_decode(pool))                       # [NP, Hkv, ps, D]
        if mode == "tensor":
            assert sc is None and mag.max() == 448.0
        elif mode == "head":
            assert sc.shape == (w.n_kv_heads,) and sc.dtype == np.float32
            assert np.all(mag.max(axis=(0, 2, 3)) == 448.0)
        else:
            assert sc.shape == (pool.shape[0], w.n_kv_heads) and sc.dtype == np.float32
            assert np.all(mag.max(axis=(2, 3)) == 448.0)
    if mode == "tensor":
        assert a["k_scale"] != 1.0
    else:
        assert a["k_scale"] == 1.0 and a["v_scale"] == 1.0

"""Helpers shared by the GPU parity tests (not collected by pytest)."""

import os

import numpy as np
import pytest

import oracle
from oracle.prologue import prologue_step, write_new_token

TOL = {"bf16": 2e-2, "fp8": 6e-2}    # max |gpu - fp64 oracle| per the method's bar


def need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import load_balanced_split_step_amd.hda as hda
    if not os.path.exists(hda.LIB_PATH):
        pytest.fail("libhda.so is not built")
    hda.load_library()


def scale_kw(inp):
    """The dequantisation-scale arguments of the oracle's attention calls."""
    return dict(k_scale=float(inp["k_scale"]), v_scale=float(inp["v_scale"]),
                scale_mode=inp.get("scale_mode", "tensor"), k_scales=inp.get("k_scales"),
                v_scales=inp.get("v_scales"))


def oracle_inputs(inp):
    """(q float64, k_pages, v_pages, extra) the oracle attends with: for a
    prologue workload, the normalised/rotated q and the pools with the new
    token written by the oracle itself; extra = (k codes, v codes, k'/scale,
    v/scale) of the new tokens."""
    if not inp["workload"].prologue:
        return oracle.bf16_to_f64(inp["q"]), inp["k_pages"], inp["v_pages"], None
    kw = scale_kw(inp)
    q_p, k_p, v, kc, vc = prologue_step(inp["q"], inp["k_new"], inp["v_new"], inp["q_norm_w"],
                                        inp["k_norm_w"], inp["seq_lens"], float(inp["rms_eps"]),
                                        float(inp["rope_theta"]), inp["kv_dtype"],
                                        block_table=inp["block_table"],
                                        page_size=inp["workload"].page_size, **kw)
    kp, vp = write_new_token(inp["k_pages"], inp["v_pages"], inp["block_table"],
                             inp["seq_lens"], kc, vc)
    Hkv = inp["workload"].n_kv_heads
    ks = oracle.slot_scales(kw["k_scale"], kw["scale_mode"], kw["k_scales"], inp["block_table"],
                            inp["seq_lens"], inp["workload"].page_size, Hkv)
    vs = oracle.slot_scales(kw["v_scale"], kw["scale_mode"], kw["v_scales"], inp["block_table"],
                            inp["seq_lens"], inp["workload"].page_size, Hkv)
    return q_p, kp, vp, (kc, vc, k_p / ks[:, :, None], v / vs[:, :, None])


def oracle_out(inp):
    q, kp, vp, _ = oracle_inputs(inp)
    return oracle.attention_reference(q, kp, vp, inp["block_table"], inp["seq_lens"],
                                      inp["kv_dtype"], float(inp["sm_scale"]), **scale_kw(inp))


def max_err(out, ref):
    got = out.detach().cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all(), "non-finite output"
    return float(np.abs(got - ref).max())

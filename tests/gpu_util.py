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


def oracle_inputs(inp):
    """(q float64, k_pages, v_pages) the oracle attends with: for a prologue
    workload, the normalised/rotated q and the pools with the new token
    written by the oracle itself."""
    if not inp["workload"].prologue:
        return oracle.bf16_to_f64(inp["q"]), inp["k_pages"], inp["v_pages"], None
    q_p, k_p, v, kc, vc = prologue_step(inp["q"], inp["k_new"], inp["v_new"], inp["q_norm_w"],
                                        inp["k_norm_w"], inp["seq_lens"], float(inp["rms_eps"]),
                                        float(inp["rope_theta"]), inp["kv_dtype"],
                                        float(inp["k_scale"]), float(inp["v_scale"]))
    kp, vp = write_new_token(inp["k_pages"], inp["v_pages"], inp["block_table"],
                             inp["seq_lens"], kc, vc)
    return q_p, kp, vp, (kc, vc, k_p / float(inp["k_scale"]), v / float(inp["v_scale"]))


def oracle_out(inp):
    q, kp, vp, _ = oracle_inputs(inp)
    return oracle.attention_reference(q, kp, vp, inp["block_table"], inp["seq_lens"],
                                      inp["kv_dtype"], float(inp["sm_scale"]),
                                      float(inp["k_scale"]), float(inp["v_scale"]))


def max_err(out, ref):
    got = out.detach().cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all(), "non-finite output"
    return float(np.abs(got - ref).max())

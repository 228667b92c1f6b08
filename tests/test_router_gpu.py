"""GPU parity of the Router GEMM against the fp64 oracle.

The weight split is bit-exact (both sides decide the bf16 codes from values
exact in float32).  The logits are checked element by element against the
exact split product x (hi + lo/256)^T within the float32 accumulation bound
(accumulation_bound), over ragged token / expert counts, hidden sizes and
split counts; two runs are bitwise equal (partials added in fixed order).
The distance to the exact fp32-weight product is printed next to that of a
plain fp32 GEMM (torch on the same device) and of a single bf16 weight.
"""

import numpy as np
import pytest
import torch

import load_balanced_split_step_amd.hda as hda
import oracle
from load_balanced_split_step_amd.workloads import ROUTER_CONFIGS, RouterWorkload, make_router_inputs
from tests.gpu_util import need_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def dev_x(x):
    return torch.from_numpy(x.view(np.int16)).cuda()


def test_split_bit_exact():
    inp = make_router_inputs(ROUTER_CONFIGS["router"])
    rw = hda.RouterWeights(inp["w"])
    torch.cuda.synchronize()
    hi, lo = oracle.split_router_weights(inp["w"])
    assert np.array_equal(rw.hi.cpu().numpy().view(np.uint16), hi)
    assert np.array_equal(rw.lo.cpu().numpy().view(np.uint16), lo)


# 1280, 4096, 16384 and 16300 tokens take the LDS-staged 128 x 128 kernel
# (with 13, 4, 1 and 1 hidden splits; 16300 x 300 with ragged token and
# expert edges); 4096 x 2080 has a hidden size the 64-wide K stages do not
# divide and runs on the register kernel
# up to 8 tokens: the one-launch kernel (whole hidden dimension per
# workgroup, one expert each), also with ragged expert counts and hidden sizes
# that leave a partial last batch of vectors
SHAPES = [(1, 256, 7168), (2, 256, 7168), (3, 300, 1024), (5, 24, 96), (7, 5, 7200),
          (8, 256, 7168), (8, 256, 8192 + 2048), (16, 256, 7168), (33, 100, 7168), (64, 256, 7168),
          (100, 256, 7168), (257, 72, 1024), (600, 256, 7168), (1280, 256, 7168),
          (4096, 256, 7168), (16384, 256, 7168), (16300, 300, 1024),
          (4096, 256, 2080)]   # hidden % 64 == 32: a large batch on the register kernel


@pytest.mark.parametrize("T,E,H", SHAPES)
def test_logits_parity(T, E, H):
    w = RouterWorkload(f"r{T}", T, H, E, seed=30 + T)
    inp = make_router_inputs(w)
    x = inp["x"]
    hi, lo = oracle.split_router_weights(inp["w"])
    ref = oracle.router_split_reference(x, hi, lo)
    bound = oracle.accumulation_bound(x, hi, lo)
    rw = hda.RouterWeights(inp["w"])
    out = rw.logits(dev_x(x))
    out2 = rw.logits(dev_x(x))
    torch.cuda.synchronize()
    o = out.cpu().numpy().astype(np.float64)
    assert torch.equal(out, out2)
    e = np.abs(o - ref)
    print(f"T={T} E={E} H={H} S={hda.hda_router_workspace_bytes(T, E, H) // max(1, 4 * T * E)}: "
          f"max |gpu - split ref| {e.max():.3e}, max err/bound {(e / bound).max():.3e}", flush=True)
    assert np.all(e <= bound)
    exact = oracle.router_reference(x, inp["w"])
    xs = torch.from_numpy(oracle.bf16_to_f64(x).astype(np.float32)).cuda()
    f32 = (xs @ torch.from_numpy(inp["w"]).cuda().T).cpu().numpy().astype(np.float64)
    b16 = oracle.bf16_to_f64(x) @ oracle.bf16_to_f64(hi).T
    print(f"   vs exact fp32-weight logits: split kernel {np.abs(o - exact).max():.3e}, "
          f"torch fp32 GEMM {np.abs(f32 - exact).max():.3e}, bf16 weight only (exact sum) "
          f"{np.abs(b16 - exact).max():.3e}", flush=True)

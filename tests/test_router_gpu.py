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
# 9 to 64 tokens: one launch, 16-expert tiles, the last workgroup of a tile
# adds the hidden-split partials (ragged expert counts, hidden sizes of 1 to
# 225 K steps; 4097 experts and hidden 32 give one range, no partials)
SHAPES = [(1, 256, 7168), (2, 256, 7168), (3, 300, 1024), (5, 24, 96), (7, 5, 7200),
          (8, 256, 7168), (8, 256, 8192 + 2048), (9, 256, 7168), (16, 256, 7168), (20, 17, 96),
          (12, 40, 32), (24, 4097, 64), (33, 100, 7168), (48, 256, 1024), (64, 256, 7168),
          (64, 300, 7200),
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
    print(f"T={T} E={E} H={H} workspace {hda.hda_router_workspace_bytes(T, E, H)} B: "
          f"max |gpu - split ref| {e.max():.3e}, max err/bound {(e / bound).max():.3e}", flush=True)
    assert np.all(e <= bound)
    exact = oracle.router_reference(x, inp["w"])
    xs = torch.from_numpy(oracle.bf16_to_f64(x).astype(np.float32)).cuda()
    f32 = (xs @ torch.from_numpy(inp["w"]).cuda().T).cpu().numpy().astype(np.float64)
    b16 = oracle.bf16_to_f64(x) @ oracle.bf16_to_f64(hi).T
    print(f"   vs exact fp32-weight logits: split kernel {np.abs(o - exact).max():.3e}, "
          f"torch fp32 GEMM {np.abs(f32 - exact).max():.3e}, bf16 weight only (exact sum) "
          f"{np.abs(b16 - exact).max():.3e}", flush=True)


def _gemm(rw, x, T, ws, out=None):
    if out is None:
        out = torch.empty((T, rw.E), dtype=torch.float32, device="cuda:0")
    hda.hda_router_gemm(x, rw.hi, rw.lo, T, rw.E, rw.H, out, ws, ws.numel(),
                        torch.cuda.current_stream())
    return out


def test_one_launch_split_any_workspace_content():
    """The one-launch split path (9 to 64 tokens) needs no cleared workspace:
    a counter word without the kernel's signature is counted by exchange on
    first use, and every call leaves the counters it used at rest.
    Workspaces filled with random bytes, with 0xff and with zeros give
    bitwise the same logits, over token counts that alternate on one
    workspace -- 100 tokens take the two-launch path, whose partial tiles
    overwrite the counters, so the next one-launch call starts from
    arbitrary words again."""
    w = RouterWorkload("r100", 100, 7168, 256, seed=77)
    inp = make_router_inputs(w)
    rw = hda.RouterWeights(inp["w"])
    x = dev_x(inp["x"])
    need = max(hda.hda_router_workspace_bytes(T, 256, 7168) for T in (16, 32, 64, 100))
    assert need > 0
    g = torch.Generator(device="cuda:0")
    g.manual_seed(5)
    fills = [torch.zeros(need, dtype=torch.uint8, device="cuda:0"),
             torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda:0"),
             torch.randint(0, 256, (need,), dtype=torch.uint8, device="cuda:0", generator=g)]
    ref = {}
    for T in (16, 32, 64, 100):
        xt = x[:T].contiguous()
        hi, lo = oracle.split_router_weights(inp["w"])
        r = oracle.router_split_reference(inp["x"][:T], hi, lo)
        bound = oracle.accumulation_bound(inp["x"][:T], hi, lo)
        ref[T] = _gemm(rw, xt, T, torch.zeros(need, dtype=torch.uint8, device="cuda:0"))
        torch.cuda.synchronize()
        assert np.all(np.abs(ref[T].cpu().numpy().astype(np.float64) - r) <= bound)
    for ws in fills:
        for T in (16, 64, 100, 32, 64, 100, 16):
            got = _gemm(rw, x[:T].contiguous(), T, ws)
            torch.cuda.synchronize()
            assert torch.equal(got, ref[T]), (T, int(ws[0]))


def test_one_launch_split_graph_replays():
    """The last arriver of each tile sets its counter back to rest, so every
    replay of a captured graph of three calls -- with eager calls on the
    same workspace in between -- gives the eager logits bit for bit."""
    T = 48
    w = RouterWorkload("r48", T, 7168, 256, seed=78)
    inp = make_router_inputs(w)
    rw = hda.RouterWeights(inp["w"])
    x = dev_x(inp["x"])
    ws = torch.empty(hda.hda_router_workspace_bytes(T, 256, 7168), dtype=torch.uint8,
                     device="cuda:0")
    eager = _gemm(rw, x, T, ws).clone()
    out = torch.zeros_like(eager)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _gemm(rw, x, T, ws, out)            # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(3):
            _gemm(rw, x, T, ws, out)
    for _ in range(4):
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
        assert torch.equal(_gemm(rw, x, T, ws), eager)
        torch.cuda.synchronize()

"""Host side of the C ABI (CPU only): the library loads and exports every
symbol include/hda.h declares, the C planners match the oracle planners
bit for bit, and argument errors come back as the documented status codes
before anything reaches the GPU."""

import os
import re

import numpy as np
import pytest

import load_balanced_split_step_amd.hda as hda
from load_balanced_split_step_amd.workloads import CONFIGS, draw_lengths
from oracle.planner import plan_dynamic, plan_static

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(hda.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return hda.load_library()


def header_functions():
    text = open(os.path.join(ROOT, "include", "hda.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hda_[a-z_]+)\s*\(", text)))


def test_exports_match_header(lib):
    names = header_functions()
    assert sorted(hda.EXPORTS) == names
    for n in names:
        assert hasattr(lib, n), n
    assert lib.hda_version() == 1


@pytest.mark.parametrize("cfg", list(CONFIGS))
@pytest.mark.parametrize("tile_len", [16, 64, 128, 256, 512])
@pytest.mark.parametrize("W", [1, 7, 64, 256, 1024])
def test_dynamic_plan_bit_exact(lib, cfg, tile_len, W):
    w = CONFIGS[cfg]
    lens = draw_lengths(w, w.seed)
    got = hda.hda_plan(lens, tile_len, W)
    want = np.array(plan_dynamic(lens.tolist(), tile_len, W).to_list(), dtype=np.int32)
    assert np.array_equal(got, want)
    assert got.size <= hda.hda_plan_capacity(len(lens), W)
    assert hda.hda_plan_validate(got, lens) == hda.HDA_OK


@pytest.mark.parametrize("cfg", list(CONFIGS))
@pytest.mark.parametrize("S", [1, 2, 4, 8, 16, 32, 64])
def test_static_plan_bit_exact(lib, cfg, S):
    w = CONFIGS[cfg]
    lens = draw_lengths(w, w.seed)
    got = hda.hda_plan_static(lens, S)
    want = np.array(plan_static(lens.tolist(), S).to_list(), dtype=np.int32)
    assert np.array_equal(got, want)
    assert got.size <= hda.hda_plan_capacity(len(lens), len(lens) * S)
    assert hda.hda_plan_validate(got, lens) == hda.HDA_OK


def test_plan_fuzz_bit_exact(lib):
    """10^4 random cases: the C++ planners and the oracle planners agree int
    for int (dynamic plans over random tile lengths and widths, static plans
    over random split counts), and every C++ plan validates."""
    rng = np.random.default_rng(1234)
    for _ in range(10000):
        B = int(rng.integers(1, 48))
        hi = int(rng.choice([3, 40, 700, 9000]))
        lens = rng.integers(1, hi + 1, size=B).astype(np.int32)
        if rng.random() < 0.5:
            tl, W = int(rng.integers(1, 300)), int(rng.integers(1, 400))
            got = hda.hda_plan(lens, tl, W)
            want = plan_dynamic(lens.tolist(), tl, W).to_list()
        else:
            S = int(rng.integers(1, 40))
            got = hda.hda_plan_static(lens, S)
            want = plan_static(lens.tolist(), S).to_list()
        assert got.tolist() == want
        assert hda.hda_plan_validate(got, lens) == hda.HDA_OK
        assert hda.hda_plan_validate(got, lens) == hda.HDA_OK


def test_plan_errors(lib):
    with pytest.raises(hda.HdaError) as e:
        hda.hda_plan(np.array([], dtype=np.int32), 16, 4)
    assert e.value.status == hda.HDA_ERR_INVALID_ARG
    for lens, tl, W in [([5, 0], 16, 4), ([5], 0, 4), ([5], 16, 0), ([-3], 16, 4)]:
        with pytest.raises(hda.HdaError) as e:
            hda.hda_plan(lens, tl, W)
        assert e.value.status == hda.HDA_ERR_INVALID_ARG
    with pytest.raises(hda.HdaError):
        hda.hda_plan_static([5], 0)
    # too-small buffer reports the size it needs
    import ctypes
    lens = np.array([17, 64, 200, 513], dtype=np.int32)
    buf = np.zeros(10, dtype=np.int32)
    n = ctypes.c_int64(0)
    st = lib.hda_plan(hda._i32p(lens), 4, 64, 4, hda._i32p(buf), 10, ctypes.byref(n))
    assert st == hda.HDA_ERR_CAPACITY and n.value == 46
    assert (buf == 0).all()                      # nothing written on failure
    assert lib.hda_plan_capacity(0, 4) == -1 and lib.hda_plan_capacity(4, 0) == -1


def corrupt(plan, lens, fn):
    p = plan.copy()
    fn(p)
    return hda.hda_plan_validate(p, lens)


def test_validate_detects_corruption(lib):
    lens = np.array([17, 64, 200, 513], dtype=np.int32)
    plan = hda.hda_plan(lens, 64, 4)
    W, N = plan[3], plan[5]
    items = 8 + W + 1
    assert hda.hda_plan_validate(plan, lens) == hda.HDA_OK
    assert hda.hda_plan_validate(plan, lens[:3]) == hda.HDA_ERR_PLAN_MISMATCH
    assert hda.hda_plan_validate(plan, lens + 1) == hda.HDA_ERR_PLAN_MISMATCH
    assert corrupt(plan, lens, lambda p: p.__setitem__(0, 2)) == hda.HDA_ERR_BAD_PLAN
    # overlap: second item of request 2 starts inside the first
    assert corrupt(plan, lens, lambda p: p.__setitem__(items + 4 * 3 + 1, 100)) == hda.HDA_ERR_BAD_PLAN
    # gap at the end of request 3
    assert corrupt(plan, lens, lambda p: p.__setitem__(items + 4 * 6 + 2, 512)) == hda.HDA_ERR_PLAN_MISMATCH
    # wrong slot
    assert corrupt(plan, lens, lambda p: p.__setitem__(items + 4 * 2 + 3, 3)) == hda.HDA_ERR_BAD_PLAN
    # slot on a single-item request
    assert corrupt(plan, lens, lambda p: p.__setitem__(items + 3, 0)) == hda.HDA_ERR_BAD_PLAN
    # wg_ptr not monotone
    assert corrupt(plan, lens, lambda p: p.__setitem__(9, 6)) == hda.HDA_ERR_BAD_PLAN
    # request index out of range
    assert corrupt(plan, lens, lambda p: p.__setitem__(items, 9)) == hda.HDA_ERR_BAD_PLAN
    # truncated
    assert hda.hda_plan_validate(plan[:-1], lens) == hda.HDA_ERR_BAD_PLAN
    assert hda.hda_plan_validate(plan[:4], lens) == hda.HDA_ERR_INVALID_ARG


def test_workspace_bytes(lib):
    lens = np.array([17, 64, 200, 513], dtype=np.int32)
    plan = hda.hda_plan(lens, 64, 4)          # P = 5
    up = lambda x: (x + 255) // 256 * 256
    q_prime = up(4 * 8 * 64 * 2) + up(4 * 8)  # prologue's q' (B x Hq x D bf16) + slot ranges
    check = up(4 * 2 * 4)                     # check words, W x Hkv int32
    assert hda.hda_workspace_bytes(plan, 8, 2, 64) == (check + up(5 * 8 * 64 * 4) + up(5 * 8 * 4)
                                                       + q_prime)
    assert hda.hda_workspace_bytes(hda.hda_plan(lens, 64, 1), 8, 2, 64) == up(2 * 4) + q_prime
    assert hda.hda_workspace_bytes(hda.hda_plan(lens, 64, 100), 8, 2, 64) > up(100 * 2 * 4)
    assert hda.hda_workspace_bytes(plan, 0, 2, 64) == -1


# --- hda_decode argument errors: all are caught on the host before launch.
# Fake, 256-byte aligned addresses stand in for device pointers; these tests
# are skipped where a GPU is visible so that no path could ever launch on them.

def _gpu_visible():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


FAKE = 0x7F0000000000


def _params(**kw):
    base = dict(batch=4, n_q_heads=8, n_kv_heads=2, head_dim=64, page_size=16,
                max_pages_per_req=33, num_pages=52, kv_dtype=hda.HDA_KV_BF16,
                sm_scale=0.125, k_scale=1.0, v_scale=1.0, prologue=0,
                workspace=FAKE + 0x100000, workspace_bytes=1 << 20)
    base.update(kw)
    return hda.hda_params(**base)


def _decode_status(lib, p, plan, **ptrs):
    import ctypes
    args = dict(q=FAKE, k=FAKE + 0x1000, v=FAKE + 0x2000, bt=FAKE + 0x3000, sl=FAKE + 0x4000,
                pd=FAKE + 0x5000, out=FAKE + 0x6000)
    args.update(ptrs)
    vp = lambda x: ctypes.c_void_p(x) if x is not None else None
    return lib.hda_decode(ctypes.byref(p), vp(args["q"]), vp(args["k"]), vp(args["v"]),
                          vp(args["bt"]), vp(args["sl"]), hda._i32p(plan), vp(args["pd"]),
                          plan.size, vp(args["out"]), None)


@pytest.mark.skipif(_gpu_visible(), reason="fake device pointers are only used without a GPU")
def test_decode_argument_errors(lib):
    lens = np.array([17, 64, 200, 513], dtype=np.int32)
    plan = hda.hda_plan(lens, 64, 4)
    E = hda
    assert _decode_status(lib, _params(), plan, q=None) == E.HDA_ERR_INVALID_ARG
    assert _decode_status(lib, _params(), plan, out=None) == E.HDA_ERR_INVALID_ARG
    assert _decode_status(lib, _params(batch=0), plan) == E.HDA_ERR_INVALID_ARG
    assert _decode_status(lib, _params(n_q_heads=7), plan) == E.HDA_ERR_INVALID_ARG
    assert _decode_status(lib, _params(sm_scale=0.0), plan) == E.HDA_ERR_INVALID_ARG
    assert _decode_status(lib, _params(k_scale=float("nan")), plan) == E.HDA_ERR_INVALID_ARG
    assert _decode_status(lib, _params(head_dim=96), plan) == E.HDA_ERR_UNSUPPORTED
    assert _decode_status(lib, _params(n_q_heads=64, n_kv_heads=2), plan) == E.HDA_ERR_UNSUPPORTED
    assert _decode_status(lib, _params(page_size=24), plan) == E.HDA_ERR_UNSUPPORTED
    assert _decode_status(lib, _params(page_size=8), plan) == E.HDA_ERR_UNSUPPORTED
    assert _decode_status(lib, _params(kv_dtype=5), plan) == E.HDA_ERR_UNSUPPORTED
    assert _decode_status(lib, _params(), plan, q=FAKE + 8) == E.HDA_ERR_INVALID_ARG
    assert _decode_status(lib, _params(prologue=1), plan) == E.HDA_ERR_INVALID_ARG
    assert _decode_status(lib, _params(batch=5), plan) == E.HDA_ERR_PLAN_MISMATCH
    assert _decode_status(lib, _params(), plan[:-1]) == E.HDA_ERR_BAD_PLAN
    bad = plan.copy(); bad[0] = 9
    assert _decode_status(lib, _params(), bad) == E.HDA_ERR_BAD_PLAN
    # workgroup item ranges: start at 0, never decrease, end at N
    W = int(plan[3])
    for pos, val in ((8, 1), (8 + W, int(plan[5]) + 1), (8 + W, int(plan[5]) - 1)):
        bad = plan.copy(); bad[pos] = val
        assert _decode_status(lib, _params(), bad) == E.HDA_ERR_BAD_PLAN, (pos, val)
    bad = plan.copy(); bad[9], bad[10] = bad[10], bad[9] - 1
    assert _decode_status(lib, _params(), bad) == E.HDA_ERR_BAD_PLAN
    # a plan in the launch arguments (no device copy) is limited in length
    long_lens = np.full(300, 100, dtype=np.int32)
    long_plan = hda.hda_plan(long_lens, 64, 64)
    assert long_plan.size > hda.HDA_PLAN_ARG_INTS
    assert _decode_status(lib, _params(batch=300), long_plan, pd=None) == E.HDA_ERR_UNSUPPORTED
    assert _decode_status(lib, _params(workspace=None), plan) == E.HDA_ERR_WORKSPACE
    assert _decode_status(lib, _params(workspace_bytes=100), plan) == E.HDA_ERR_WORKSPACE
    # scale granularity
    assert _decode_status(lib, _params(scale_mode=3), plan) == E.HDA_ERR_INVALID_ARG
    assert _decode_status(lib, _params(scale_mode=E.HDA_SCALE_HEAD), plan) == E.HDA_ERR_INVALID_ARG
    assert _decode_status(lib, _params(scale_mode=E.HDA_SCALE_HEAD, k_scales=FAKE + 0x7000),
                          plan) == E.HDA_ERR_INVALID_ARG
    assert _decode_status(lib, _params(scale_mode=E.HDA_SCALE_PAGE, k_scales=FAKE + 0x7000,
                                       v_scales=FAKE + 0x8000), plan) == E.HDA_ERR_UNSUPPORTED
    assert _decode_status(lib, _params(reserved0=1), plan) == E.HDA_ERR_INVALID_ARG
    # native-fp8 products and dim-major V pages
    fp8n = dict(kv_dtype=E.HDA_KV_FP8_E4M3, head_dim=128, page_size=64, math=E.HDA_MATH_FP8,
                v_layout=E.HDA_V_DIM_MAJOR)
    assert _decode_status(lib, _params(math=2), plan) == E.HDA_ERR_INVALID_ARG
    assert _decode_status(lib, _params(v_layout=2), plan) == E.HDA_ERR_INVALID_ARG
    assert _decode_status(lib, _params(**dict(fp8n, kv_dtype=E.HDA_KV_BF16)), plan) == E.HDA_ERR_UNSUPPORTED
    assert _decode_status(lib, _params(**dict(fp8n, v_layout=0)), plan) == E.HDA_ERR_UNSUPPORTED
    assert _decode_status(lib, _params(**dict(fp8n, head_dim=64)), plan) == E.HDA_ERR_UNSUPPORTED
    assert _decode_status(lib, _params(**dict(fp8n, page_size=32)), plan) == E.HDA_ERR_UNSUPPORTED
    assert _decode_status(lib, _params(**dict(fp8n, scale_mode=E.HDA_SCALE_PAGE, k_scales=FAKE + 0x7000,
                                              v_scales=FAKE + 0x8000)), plan) == E.HDA_ERR_UNSUPPORTED
    assert _decode_status(lib, _params(v_layout=E.HDA_V_DIM_MAJOR), plan) == E.HDA_ERR_UNSUPPORTED
    for s in (0, -1, -2, -3, -4, -5, -6, -7):
        assert lib.hda_status_string(s)


def test_header_constants_match_binding():
    """Every #define of the header that the binding mirrors has the same value."""
    import re
    text = open(os.path.join(ROOT, "include", "hda.h")).read()
    defs = {m.group(1): int(m.group(2)) for m in
            re.finditer(r"#define\s+(HDA_\w+)\s+\(?(-?\d+)\)?", text)}
    mirrored = [k for k in dir(hda) if k.startswith("HDA_") and isinstance(getattr(hda, k), int)]
    assert len(mirrored) >= 13
    for k in mirrored:
        assert defs[k] == getattr(hda, k), k
    assert defs["HDA_PLAN_HEADER_INTS"] == hda.PLAN_HEADER_INTS


def test_workspace_bound(lib):
    up = lambda x: (x + 255) // 256 * 256
    assert hda.hda_workspace_bytes_bound(4, 8, 8, 64) == (up(8 * 8 * 4) + up(11 * 8 * 64 * 4)
                                                          + up(11 * 8 * 4) + up(4 * 8 * 64 * 2)
                                                          + up(4 * 8))
    assert hda.hda_workspace_bytes_bound(0, 8, 8, 64) == -1
    # the bound covers every plan over the same batch and workgroup count
    rng = np.random.default_rng(9)
    for _ in range(200):
        B, W = int(rng.integers(1, 40)), int(rng.integers(1, 200))
        lens = rng.integers(1, 3000, size=B).astype(np.int32)
        plan = hda.hda_plan(lens, int(rng.integers(1, 300)), W)
        assert hda.hda_workspace_bytes(plan, 8, 2, 128) <= hda.hda_workspace_bytes_bound(B, W, 8, 128)


@pytest.mark.skipif(_gpu_visible(), reason="fake device pointers are only used without a GPU")
def test_decode_auto_and_plan_device_argument_errors(lib):
    import ctypes
    E = hda
    vp = ctypes.c_void_p

    def auto(p, tl=64, W=4, **ptrs):
        a = dict(q=FAKE, k=FAKE + 0x1000, v=FAKE + 0x2000, bt=FAKE + 0x3000, sl=FAKE + 0x4000,
                 out=FAKE + 0x6000)
        a.update(ptrs)
        f = lambda x: vp(x) if x is not None else None
        return lib.hda_decode_auto(ctypes.byref(p), f(a["q"]), f(a["k"]), f(a["v"]), f(a["bt"]),
                                   f(a["sl"]), tl, W, f(a["out"]), None)

    assert auto(_params(), sl=None) == E.HDA_ERR_INVALID_ARG
    assert auto(_params(), tl=0) == E.HDA_ERR_INVALID_ARG
    assert auto(_params(), W=0) == E.HDA_ERR_INVALID_ARG
    assert auto(_params(head_dim=80)) == E.HDA_ERR_UNSUPPORTED
    assert auto(_params(workspace=None)) == E.HDA_ERR_WORKSPACE
    assert auto(_params(workspace_bytes=1000), W=64) == E.HDA_ERR_WORKSPACE
    assert lib.hda_plan_device(None, 4, 64, 4, vp(FAKE), 1000, None) == E.HDA_ERR_INVALID_ARG
    assert lib.hda_plan_device(vp(FAKE), 4, 0, 4, vp(FAKE), 1000, None) == E.HDA_ERR_INVALID_ARG
    assert lib.hda_plan_device(vp(FAKE), 4, 64, 4, vp(FAKE), 10, None) == E.HDA_ERR_CAPACITY


# ---- multi-token (prefill) host entry points ----

def test_prefill_rows_per_block(lib):
    assert hda.hda_prefill_rows_per_block(64, 8) == 2
    assert hda.hda_prefill_rows_per_block(8, 2) == 4
    assert hda.hda_prefill_rows_per_block(16, 16) == 16
    assert hda.hda_prefill_rows_per_block(16, 1) == 1
    assert hda.hda_prefill_rows_per_block(34, 2) == -1
    assert hda.hda_prefill_rows_per_block(7, 2) == -1


def test_prefill_rows_bit_exact(lib):
    import oracle
    golden = os.path.join(ROOT, "tests", "golden", "prefill_rows.txt")
    g = {}
    for line in open(golden):
        if line.strip() and not line.startswith("#"):
            k, *v = line.split()
            g.setdefault(k, []).append([int(x) if x.lstrip("-").isdigit() else x for x in v])
    rows, row_lens = hda.hda_prefill_rows(g["q_lens"][0], g["kv_lens"][0], g["rows_per_block"][0][0])
    assert rows.tolist() == g["row"] and row_lens.tolist() == g["extents"][0]
    plan = hda.hda_plan(row_lens, 4, 3)
    assert plan[:8].tolist() == g["header"][0]
    rng = np.random.default_rng(11)
    for _ in range(500):
        B = int(rng.integers(1, 40))
        kv = rng.integers(1, int(rng.choice([10, 500, 50000])), size=B).astype(np.int32)
        ql = np.minimum(rng.integers(1, int(rng.choice([3, 70, 2000])), size=B), kv).astype(np.int32)
        qb = int(rng.choice([1, 2, 4, 8, 16]))
        rows, row_lens = hda.hda_prefill_rows(ql, kv, qb)
        want, ext = oracle.prefill_rows(ql, kv, qb)
        assert [tuple(r) for r in rows.tolist()] == want and row_lens.tolist() == ext


def test_prefill_rows_errors(lib):
    import ctypes
    n = ctypes.c_int64(0)
    ql = np.array([3, 5], np.int32)
    kv = np.array([10, 4], np.int32)           # q_len > kv_len for request 1
    st = lib.hda_prefill_rows(hda._i32p(ql), hda._i32p(kv), 2, 2, None, None, 0, ctypes.byref(n))
    assert st == hda.HDA_ERR_INVALID_ARG
    kv = np.array([10, 5], np.int32)
    st = lib.hda_prefill_rows(hda._i32p(ql), hda._i32p(kv), 2, 2, None, None, 0, ctypes.byref(n))
    assert st == hda.HDA_ERR_CAPACITY and n.value == 2 + 3
    rows = np.empty((4, 4), np.int32)
    lens = np.empty(4, np.int32)
    st = lib.hda_prefill_rows(hda._i32p(ql), hda._i32p(kv), 2, 2, hda._i32p(rows), hda._i32p(lens),
                              4, ctypes.byref(n))
    assert st == hda.HDA_ERR_CAPACITY and n.value == 5
    st = lib.hda_prefill_rows(hda._i32p(ql), hda._i32p(kv), 2, 0, None, None, 0, ctypes.byref(n))
    assert st == hda.HDA_ERR_INVALID_ARG


def test_prefill_block_rows(lib):
    """Tiles of 16/g rows: the smallest power of two (at most 16) covering the
    mean query run."""
    f = hda.hda_prefill_block_rows
    assert f([1, 1, 1], 64, 8) == 2                    # decode rows: one tile
    assert f([2, 2], 64, 8) == 2
    assert f([3, 2], 64, 8) == 4                       # mean 2.5 rows: 2 tiles
    assert f([4] * 32, 64, 8) == 4                     # speculative checks of 4
    assert f([5, 4], 64, 8) == 8                       # mean 4.5 rows: 3 tiles -> 4
    assert f([16, 16], 64, 8) == 16                    # 8 tiles
    assert f([20, 12], 64, 8) == 16                    # mean 16 rows: 8 tiles
    assert f([21, 12], 64, 8) == 32                    # mean 16.5 rows: 9 tiles -> 16
    assert f([128, 100], 64, 8) == 32                  # capped at 16 tiles
    assert f([20, 3, 33], 32, 2) == 16                 # group 16: 1-row tiles, mean 18.7 -> 16
    assert f([1], 32, 2) == 1
    assert f([16], 16, 16) == 16                       # group 1: 16-row tiles
    assert f([17], 16, 16) == 32
    assert f([0, 4], 64, 8) == -1
    assert f([4], 7, 2) == -1
    assert f([], 64, 8) == -1


def test_prefill_workspace_bytes(lib):
    up = lambda x: (x + 255) // 256 * 256
    rows, row_lens = hda.hda_prefill_rows([3, 1, 5], [10, 1, 5], 2)
    plan = hda.hda_plan(row_lens, 4, 3)
    P = int(plan[6])
    assert P == 2
    c = up(3 * 8 * 4)                         # check words, W x Hkv int32
    assert hda.hda_prefill_workspace_bytes(plan, 64, 8, 128, 2) == c + up(P * 2 * 64 * 128 * 4) + up(P * 2 * 64 * 4)
    assert hda.hda_prefill_workspace_bytes(plan, 64, 8, 128, 8) == c + up(P * 8 * 64 * 128 * 4) + up(P * 8 * 64 * 4)
    assert hda.hda_prefill_workspace_bytes(plan, 64, 8, 128, 32) == c + up(P * 32 * 64 * 128 * 4) + up(P * 32 * 64 * 4)
    assert hda.hda_prefill_workspace_bytes(plan, 64, 8, 128, 33) == -1     # above 16 x 16/g
    assert hda.hda_prefill_workspace_bytes(plan, 64, 3, 128, 2) == -1


@pytest.mark.skipif(_gpu_visible(), reason="fake device pointers are only used without a GPU")
def test_prefill_argument_errors(lib):
    import ctypes
    E = hda
    q_lens, kv_lens = np.array([3, 1, 5], np.int32), np.array([10, 1, 5], np.int32)
    rows, row_lens = hda.hda_prefill_rows(q_lens, kv_lens, 2)
    plan = hda.hda_plan(row_lens, 4, 3)
    vp = lambda x: ctypes.c_void_p(x) if x is not None else None

    def call(p, rows=rows, plan=plan, n_q=9, **kw):
        a = dict(q=FAKE, k=FAKE + 0x1000, v=FAKE + 0x2000, bt=FAKE + 0x3000, kv=FAKE + 0x4000,
                 rd=FAKE + 0x5000, pd=FAKE + 0x6000, out=FAKE + 0x7000)
        a.update(kw)
        rows = np.ascontiguousarray(rows, np.int32)
        return lib.hda_prefill(ctypes.byref(p), vp(a["q"]), vp(a["k"]), vp(a["v"]), vp(a["bt"]),
                               vp(a["kv"]), n_q, hda._i32p(rows), vp(a["rd"]), hda._i32p(plan),
                               vp(a["pd"]), plan.size, vp(a["out"]), None)

    base = dict(batch=3, n_q_heads=64, n_kv_heads=8, head_dim=128, page_size=16)
    assert call(_params(**base), q=None) == E.HDA_ERR_INVALID_ARG
    assert call(_params(**base, prologue=1, q_norm_w=FAKE, k_norm_w=FAKE, k_new=FAKE,
                        v_new=FAKE, rope_theta=1e6)) == E.HDA_ERR_UNSUPPORTED
    assert call(_params(**dict(base, kv_dtype=E.HDA_KV_FP8_E4M3, math=E.HDA_MATH_FP8,
                               v_layout=E.HDA_V_DIM_MAJOR, page_size=64))) == E.HDA_ERR_UNSUPPORTED
    assert call(_params(**base), n_q=8) == E.HDA_ERR_INVALID_ARG        # last block past n_q
    bad = rows.copy(); bad[0, 2] = 33                                    # 33 rows > 16 x 2 per block
    assert call(_params(**base), rows=bad, n_q=40) == E.HDA_ERR_INVALID_ARG
    bad = rows.copy(); bad[1, 0] = 3                                     # request out of range
    assert call(_params(**base), rows=bad) == E.HDA_ERR_INVALID_ARG
    assert call(_params(**base), plan=plan[:-1]) == E.HDA_ERR_BAD_PLAN
    # workgroup item ranges: from 0, non-decreasing, ending at N
    N = int(plan[5])
    for k, v in [(8, 1), (9, N + 5), (8 + 3, N - 1)]:
        bad = plan.copy(); bad[k] = v
        assert call(_params(**base), plan=bad) == E.HDA_ERR_BAD_PLAN, (k, v)
    assert call(_params(**base, workspace=None)) == E.HDA_ERR_WORKSPACE
    assert call(_params(**base, workspace_bytes=64)) == E.HDA_ERR_WORKSPACE


@pytest.mark.skipif(_gpu_visible(), reason="fake device pointers are only used without a GPU")
def test_check_and_coverage_argument_errors(lib):
    import ctypes
    flags = ctypes.c_int32(0)
    chk = lambda p, W: lib.hda_decode_check(ctypes.byref(p) if p is not None else None, W,
                                            ctypes.byref(flags), None)
    assert chk(None, 4) == hda.HDA_ERR_INVALID_ARG
    assert chk(_params(workspace=None), 4) == hda.HDA_ERR_INVALID_ARG
    assert chk(_params(), 0) == hda.HDA_ERR_INVALID_ARG
    assert chk(_params(workspace_bytes=4 * 2 * 4 - 1), 4) == hda.HDA_ERR_INVALID_ARG  # W x Hkv words
    lens = np.array([17, 64, 200, 513], dtype=np.int32)
    plan = hda.hda_plan(lens, 64, 4)
    vp = ctypes.c_void_p

    def cov(visits, plan_dev):
        return lib.hda_decode_coverage(ctypes.byref(_params()), vp(FAKE), vp(FAKE + 0x1000),
                                       vp(FAKE + 0x2000), vp(FAKE + 0x3000), vp(FAKE + 0x4000),
                                       hda._i32p(plan), plan_dev, plan.size, vp(FAKE + 0x5000),
                                       visits, None)
    assert cov(None, vp(FAKE + 0x6000)) == hda.HDA_ERR_INVALID_ARG
    assert cov(vp(FAKE + 0x7000), None) == hda.HDA_ERR_INVALID_ARG


def test_router_workspace_bytes_shapes(lib):
    """The launch-shape arithmetic on the host: every accepted shape gives a
    whole number of partial tiles, small and odd hidden sizes included --
    none up to 8 tokens (one workgroup per expert over the whole hidden
    dimension); from 9 to 64 tokens 8-byte counters for the ceil(E/16)
    expert tiles (rounded up to 256 bytes) plus S tiles of 16 MB x 16 floats
    each, MB = 1, 2 or 4 for up to 16, 32 or 64 tokens, S at most H/32;
    beyond, S x T x E x 4 bytes with S at most ceil(H/128) -- and rejected
    shapes give -1."""
    for T in (1, 5, 8, 9, 16, 17, 33, 64, 65, 100, 1000, 20000):
        for E in (1, 24, 64, 256):
            for H in (32, 64, 96, 128, 160, 1024, 7168):
                n = hda.hda_router_workspace_bytes(T, E, H)
                assert n >= 0
                if T <= 8:
                    assert n == 0
                elif T <= 64:
                    tiles = -(-E // 16)
                    tm = 16 if T <= 16 else 32 if T <= 32 else 64
                    if n:
                        c = -(-tiles * 8 // 256) * 256
                        assert (n - c) % (tiles * tm * 16 * 4) == 0
                        S = (n - c) // (tiles * tm * 16 * 4)
                        assert 2 <= S <= H // 32
                    else:
                        assert tiles >= 256 or H == 32
                else:
                    assert n % (4 * T * E) == 0
                    S = n // (4 * T * E)
                    assert S == 0 or 2 <= S <= -(-H // 128)
    assert hda.hda_router_workspace_bytes(4, 8, 48) == -1
    assert hda.hda_router_workspace_bytes(0, 8, 64) == -1
    assert hda.hda_router_workspace_bytes(4, 8, 0) == -1


@pytest.mark.skipif(_gpu_visible(), reason="fake device pointers are only used without a GPU")
def test_router_argument_errors(lib):
    import ctypes
    E = hda
    vp = ctypes.c_void_p

    def call(x=FAKE, hi=FAKE + 0x1000, lo=FAKE + 0x2000, T=8, Ex=16, H=64, out=FAKE + 0x3000,
             ws=None, wsb=0):
        return lib.hda_router_gemm(vp(x) if x else None, vp(hi) if hi else None,
                                   vp(lo) if lo else None, T, Ex, H, vp(out) if out else None,
                                   vp(ws) if ws else None, wsb, None)

    assert call(x=None) == E.HDA_ERR_INVALID_ARG
    assert call(out=None) == E.HDA_ERR_INVALID_ARG
    assert call(T=0) == E.HDA_ERR_INVALID_ARG
    assert call(H=48) == E.HDA_ERR_UNSUPPORTED
    assert call(x=FAKE + 8) == E.HDA_ERR_INVALID_ARG                 # not 16-byte aligned
    assert call(T=1 << 20, H=1024) == E.HDA_ERR_UNSUPPORTED          # beyond 32-bit offsets
    need = hda.hda_router_workspace_bytes(8, 16, 64)
    if need > 0:
        assert call() == E.HDA_ERR_WORKSPACE
        assert call(ws=FAKE + 0x4000, wsb=need - 4) == E.HDA_ERR_WORKSPACE
    # 16 tokens take the one-launch split path: its counters and partial
    # tiles need a workspace, 16-byte aligned
    need16 = hda.hda_router_workspace_bytes(16, 16, 64)
    assert need16 > 0
    assert call(T=16) == E.HDA_ERR_WORKSPACE
    assert call(T=16, ws=FAKE + 0x4000, wsb=need16 - 1) == E.HDA_ERR_WORKSPACE
    assert call(T=16, ws=FAKE + 0x4008, wsb=need16) == E.HDA_ERR_INVALID_ARG
    assert lib.hda_router_split_weights(None, 10, vp(FAKE), vp(FAKE), None) == E.HDA_ERR_INVALID_ARG
    assert lib.hda_router_split_weights(vp(FAKE), 0, vp(FAKE), vp(FAKE), None) == E.HDA_ERR_INVALID_ARG


def test_read_probe_argument_errors(lib):
    """The read probe rejects bad arguments on the host, before any launch."""
    import ctypes
    vp = ctypes.c_void_p
    assert lib.hda_read_probe(None, 1024, 4, vp(FAKE), None) == hda.HDA_ERR_INVALID_ARG
    assert lib.hda_read_probe(vp(FAKE), 1024, 4, None, None) == hda.HDA_ERR_INVALID_ARG
    assert lib.hda_read_probe(vp(FAKE), 1000, 4, vp(FAKE), None) == hda.HDA_ERR_INVALID_ARG
    assert lib.hda_read_probe(vp(FAKE), 0, 4, vp(FAKE), None) == hda.HDA_ERR_INVALID_ARG
    assert lib.hda_read_probe(vp(FAKE), 1024, 0, vp(FAKE), None) == hda.HDA_ERR_INVALID_ARG
    assert lib.hda_read_probe(vp(FAKE + 8), 1024, 4, vp(FAKE), None) == hda.HDA_ERR_INVALID_ARG


def test_plan_upload_argument_errors(lib):
    """The plan upload rejects bad arguments on the host, before any launch."""
    import ctypes
    vp = ctypes.c_void_p
    plan = np.arange(16, dtype=np.int32)
    pp = plan.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    assert lib.hda_plan_upload(None, 16, vp(FAKE), None) == hda.HDA_ERR_INVALID_ARG
    assert lib.hda_plan_upload(pp, 16, None, None) == hda.HDA_ERR_INVALID_ARG
    assert lib.hda_plan_upload(pp, 0, vp(FAKE), None) == hda.HDA_ERR_INVALID_ARG
    assert lib.hda_plan_upload(pp, -3, vp(FAKE), None) == hda.HDA_ERR_INVALID_ARG
    assert lib.hda_plan_upload(pp, 16, vp(FAKE + 2), None) == hda.HDA_ERR_INVALID_ARG
    with pytest.raises(ValueError):
        hda.hda_plan_upload(plan, 0, plan_len=17)


def test_launch_config(lib):
    """hda_launch_config: on the extreme mix, 63 workgroups (only the long
    request split); on the uniform mix 32 (one request per workgroup, no
    partial slots); in general, by brute force with the oracle planner's
    partial-slot count: the widest of the widths with the fewest partial
    slots among those whose busiest compute unit (ceil(W Hkv / 256)
    workgroups of ceil(T / W) tiles) holds at most 1/32 more tiles than the
    least possible."""
    import oracle
    lens = np.array([131072] + [4096] * 31, np.int32)
    assert hda.launch_config(lens, 8) == (128, 63)
    assert oracle.plan_dynamic(lens.tolist(), 128, 63).n_partials == 32
    assert hda.launch_config(np.full(32, 4096, np.int32), 8) == (128, 32)
    assert oracle.plan_dynamic([4096] * 32, 128, 32).n_partials == 0
    rng = np.random.default_rng(12)
    for _ in range(200):
        B = int(rng.integers(1, 70))
        lens = np.exp(rng.uniform(0, np.log(40000), size=B)).astype(np.int32) + 1
        hkv = int(rng.choice([1, 2, 4, 8, 16]))
        tl, W = hda.launch_config(lens, hkv)
        T = int(sum(-(-int(x) // tl) for x in lens))
        wmax = max(1, min(T, 512 // hkv))
        unit = {w: -(-w * hkv // 256) * -(-T // w) for w in range(1, wmax + 1)}
        least = min(unit.values())
        cands = [w for w in unit if unit[w] * 32 <= least * 33]
        P = {w: oracle.plan_dynamic(lens.tolist(), tl, w).n_partials for w in cands}
        best = min(P.values())
        assert P[W] == best and W == max(w for w in cands if P[w] == best), (lens, hkv, W)
    f = lambda *a: lib.hda_launch_config(*a)
    import ctypes
    out = ctypes.c_int32(0)
    lens = np.array([5, 6], np.int32)
    assert f(hda._i32p(lens), 2, 0, 256, 2, 128, ctypes.byref(out)) == hda.HDA_ERR_INVALID_ARG
    assert f(hda._i32p(lens), 2, 8, 256, 2, 0, ctypes.byref(out)) == hda.HDA_ERR_INVALID_ARG
    assert f(hda._i32p(lens), 0, 8, 256, 2, 128, ctypes.byref(out)) == hda.HDA_ERR_INVALID_ARG
    assert f(hda._i32p(lens), 2, 8, 256, 2, 128, None) == hda.HDA_ERR_INVALID_ARG


def test_one_hip_runtime_in_process():
    """Loading libhda.so through the binding leaves one HIP runtime mapped
    (torch's): the binding imports torch before it opens the library."""
    import subprocess
    import sys
    code = ("import load_balanced_split_step_amd.hda as h; h.load_library(); "
            "print(sorted({l.split()[-1] for l in open('/proc/self/maps') if 'amdhip64' in l}))")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                         check=True).stdout.strip()
    libs = eval(out)
    assert len(libs) == 1, libs

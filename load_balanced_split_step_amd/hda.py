"""ctypes binding of libhda.so (include/hda.h).

Argument marshalling only: every step of the decode path runs in the HIP
library.  PyTorch supplies device memory and streams.  Importing this module
does not load the library; the first call does, and raises if libhda.so is
missing -- there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhda.so")

HDA_OK = 0
HDA_ERR_INVALID_ARG = -1
HDA_ERR_CAPACITY = -2
HDA_ERR_UNSUPPORTED = -3
HDA_ERR_PLAN_MISMATCH = -4
HDA_ERR_HIP = -5
HDA_ERR_WORKSPACE = -6
HDA_ERR_BAD_PLAN = -7

HDA_KV_BF16 = 0
HDA_KV_FP8_E4M3 = 1
HDA_SCALE_TENSOR = 0
HDA_SCALE_HEAD = 1
HDA_SCALE_PAGE = 2
SCALE_MODES = {"tensor": HDA_SCALE_TENSOR, "head": HDA_SCALE_HEAD, "page": HDA_SCALE_PAGE}
HDA_MATH_BF16 = 0
HDA_MATH_FP8 = 1
HDA_V_TOKEN_MAJOR = 0
HDA_V_DIM_MAJOR = 1
HDA_NOALLOC_WORKSPACE_BYTES = 16777216   # hda_decode_noalloc's own workspace
HDA_CHECK_PAST_LEN = 1         # device check bits (hda_decode_check)
HDA_CHECK_SHORT = 2
HDA_PREFILL_MAX_TILES = 16
HDA_PLAN_UPLOAD_CHUNK = 1000   # plan ints per hda_plan_upload launch
HDA_PLAN_ARG_INTS = 896        # longest plan hda_decode takes in its launch arguments
PLAN_HEADER_INTS = 8

# every symbol include/hda.h declares
EXPORTS = ("hda_plan_capacity", "hda_plan", "hda_launch_config", "hda_plan_static",
           "hda_plan_validate",
           "hda_workspace_bytes", "hda_decode", "hda_decode_noalloc", "hda_decode_coverage",
           "hda_decode_check",
           "hda_decode_auto", "hda_workspace_bytes_bound",
           "hda_plan_device", "hda_plan_upload", "hda_prefill_rows_per_block", "hda_prefill_block_rows",
           "hda_prefill_rows",
           "hda_prefill_workspace_bytes", "hda_prefill", "hda_router_split_weights",
           "hda_router_workspace_bytes", "hda_router_gemm", "hda_read_probe", "hda_status_string",
           "hda_version",
           "hda_params_bytes")


class HdaError(RuntimeError):
    def __init__(self, status, what=""):
        self.status = status
        super().__init__(f"{what}: {hda_status_string(status)} ({status})")


class hda_params(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_pages_per_req", ctypes.c_int32),
        ("num_pages", ctypes.c_int64),
        ("kv_dtype", ctypes.c_int32),
        ("sm_scale", ctypes.c_float),
        ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float),
        ("prologue", ctypes.c_int32),
        ("rms_eps", ctypes.c_float),
        ("rope_theta", ctypes.c_float),
        ("q_norm_w", ctypes.c_void_p),
        ("k_norm_w", ctypes.c_void_p),
        ("k_new", ctypes.c_void_p),
        ("v_new", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_int64),
        ("split_event", ctypes.c_void_p),
        ("scale_mode", ctypes.c_int32),
        ("math", ctypes.c_int32),
        ("k_scales", ctypes.c_void_p),
        ("v_scales", ctypes.c_void_p),
        ("v_layout", ctypes.c_int32),
        ("reserved0", ctypes.c_int32),
    ]


_lib = None


def load_library(path: Optional[str] = None):
    """Load libhda.so (once).  Raises OSError if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise OSError(f"libhda.so not found at {path}; run __graft_entry__.build()")
    # torch ships its own HIP runtime; loaded first, it also serves
    # libhda.so's libamdhip64 dependency.  Loaded after libhda.so, it would be
    # a second runtime in the process, and launches on torch's streams
    # would fail.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    pi32 = ctypes.POINTER(ctypes.c_int32)
    pi64 = ctypes.POINTER(ctypes.c_int64)
    sig = {
        "hda_plan_capacity": (i64, [i32, i32]),
        "hda_plan": (ctypes.c_int, [pi32, i32, i32, i32, pi32, i64, pi64]),
        "hda_plan_static": (ctypes.c_int, [pi32, i32, i32, pi32, i64, pi64]),
        "hda_launch_config": (ctypes.c_int, [pi32, i32, i32, i32, i32, i32, pi32]),
        "hda_plan_validate": (ctypes.c_int, [pi32, i64, pi32, i32]),
        "hda_workspace_bytes": (i64, [pi32, i64, i32, i32, i32]),
        "hda_decode": (ctypes.c_int, [ctypes.POINTER(hda_params), vp, vp, vp, vp, vp, pi32, vp,
                                      i64, vp, vp]),
        "hda_decode_noalloc": (ctypes.c_int, [ctypes.POINTER(hda_params), vp, vp, vp, vp, vp,
                                              pi32, vp, i64, vp, vp]),
        "hda_decode_coverage": (ctypes.c_int, [ctypes.POINTER(hda_params), vp, vp, vp, vp, vp,
                                               pi32, vp, i64, vp, vp, vp]),
        "hda_decode_check": (ctypes.c_int, [ctypes.POINTER(hda_params), i32, pi32, vp]),
        "hda_decode_auto": (ctypes.c_int, [ctypes.POINTER(hda_params), vp, vp, vp, vp, vp, i32, i32,
                                           vp, vp]),
        "hda_workspace_bytes_bound": (i64, [i32, i32, i32, i32]),
        "hda_plan_device": (ctypes.c_int, [vp, i32, i32, i32, vp, i64, vp]),
        "hda_plan_upload": (ctypes.c_int, [pi32, i64, vp, vp]),
        "hda_prefill_rows_per_block": (i32, [i32, i32]),
        "hda_prefill_block_rows": (i32, [pi32, i32, i32, i32]),
        "hda_prefill_rows": (ctypes.c_int, [pi32, pi32, i32, i32, pi32, pi32, i64, pi64]),
        "hda_prefill_workspace_bytes": (i64, [pi32, i64, i32, i32, i32, i32]),
        "hda_prefill": (ctypes.c_int, [ctypes.POINTER(hda_params), vp, vp, vp, vp, vp, i32, pi32,
                                       vp, pi32, vp, i64, vp, vp]),
        "hda_router_split_weights": (ctypes.c_int, [vp, i64, vp, vp, vp]),
        "hda_router_workspace_bytes": (i64, [i32, i32, i32]),
        "hda_router_gemm": (ctypes.c_int, [vp, vp, vp, i32, i32, i32, vp, vp, i64, vp]),
        "hda_read_probe": (ctypes.c_int, [vp, i64, i32, vp, vp]),
        "hda_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "hda_version": (ctypes.c_int, []),
        "hda_params_bytes": (i64, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.hda_params_bytes() != ctypes.sizeof(hda_params):
        raise OSError("hda_params layout differs between libhda.so and this binding")
    _lib = lib
    return lib


def _i32p(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _lens(seq_lens):
    a = np.ascontiguousarray(seq_lens, dtype=np.int32)
    if a.ndim != 1:
        raise ValueError("seq_lens must be 1-D")
    return a


def hda_status_string(status: int) -> str:
    return load_library().hda_status_string(int(status)).decode()


def hda_version() -> int:
    return load_library().hda_version()


def hda_plan_capacity(batch: int, n_workgroups: int) -> int:
    return load_library().hda_plan_capacity(int(batch), int(n_workgroups))


def _plan_call(fn, lens, *args):
    lib = load_library()
    n = ctypes.c_int64(0)
    st = fn(_i32p(lens), len(lens), *args, None, 0, ctypes.byref(n))
    if st not in (HDA_OK, HDA_ERR_CAPACITY, HDA_ERR_INVALID_ARG):
        raise HdaError(st, fn.__name__)
    if st == HDA_ERR_INVALID_ARG and n.value == 0:
        raise HdaError(st, fn.__name__)
    plan = np.empty(n.value, dtype=np.int32)
    st = fn(_i32p(lens), len(lens), *args, _i32p(plan), plan.size, ctypes.byref(n))
    if st != HDA_OK:
        raise HdaError(st, fn.__name__)
    return plan


def hda_plan(seq_lens, tile_len: int, n_workgroups: int) -> np.ndarray:
    """Dynamic tile plan (int32 array) for the host lengths."""
    lib = load_library()
    return _plan_call(lib.hda_plan, _lens(seq_lens), int(tile_len), int(n_workgroups))


def hda_plan_into(seq_lens, tile_len: int, n_workgroups: int, out: np.ndarray) -> int:
    """Dynamic plan written into a caller buffer (int32, e.g. a pinned host
    tensor's numpy view); returns the number of ints used.  No allocation."""
    lib = load_library()
    lens = _lens(seq_lens)
    n = ctypes.c_int64(0)
    st = lib.hda_plan(_i32p(lens), len(lens), int(tile_len), int(n_workgroups), _i32p(out),
                      out.size, ctypes.byref(n))
    if st != HDA_OK:
        raise HdaError(st, "hda_plan")
    return n.value


def hda_plan_static(seq_lens, n_splits: int) -> np.ndarray:
    """Static split baseline plan (int32 array)."""
    lib = load_library()
    return _plan_call(lib.hda_plan_static, _lens(seq_lens), int(n_splits))


def hda_plan_validate(plan, seq_lens) -> int:
    """Status code of hda_plan_validate (HDA_OK when the plan fits the lengths)."""
    lib = load_library()
    plan = np.ascontiguousarray(plan, dtype=np.int32)
    lens = _lens(seq_lens)
    return lib.hda_plan_validate(_i32p(plan), plan.size, _i32p(lens), len(lens))


def hda_workspace_bytes(plan, n_q_heads: int, n_kv_heads: int, head_dim: int) -> int:
    lib = load_library()
    plan = np.ascontiguousarray(plan, dtype=np.int32)
    return lib.hda_workspace_bytes(_i32p(plan), plan.size, int(n_q_heads), int(n_kv_heads),
                                   int(head_dim))


def hda_decode(params: hda_params, q, k_pages, v_pages, block_table, seq_lens, plan_host,
               plan_dev, out, stream=None) -> None:
    """Enqueue one decode step.  q, k_pages, ... are device pointers (ints) or
    torch tensors; plan_host is the host int32 array; stream is a raw
    hipStream_t (int) or a torch stream, default the current torch stream."""
    lib = load_library()
    plan_host = np.ascontiguousarray(plan_host, dtype=np.int32)
    st = lib.hda_decode(ctypes.byref(params), _ptr(q), _ptr(k_pages), _ptr(v_pages),
                        _ptr(block_table), _ptr(seq_lens), _i32p(plan_host), _ptr(plan_dev),
                        plan_host.size, _ptr(out), _stream(stream))
    if st != HDA_OK:
        raise HdaError(st, "hda_decode")


def hda_decode_noalloc(params: hda_params, q, k_pages, v_pages, block_table, seq_lens, plan_host,
                       plan_dev, out, stream=None) -> None:
    """Enqueue one decode step with the library's own device workspace
    (params.workspace is ignored; see include/hda.h)."""
    lib = load_library()
    plan_host = np.ascontiguousarray(plan_host, dtype=np.int32)
    st = lib.hda_decode_noalloc(ctypes.byref(params), _ptr(q), _ptr(k_pages), _ptr(v_pages),
                                _ptr(block_table), _ptr(seq_lens), _i32p(plan_host),
                                _ptr(plan_dev), plan_host.size, _ptr(out), _stream(stream))
    if st != HDA_OK:
        raise HdaError(st, "hda_decode_noalloc")


def hda_decode_coverage(params: hda_params, q, k_pages, v_pages, block_table, seq_lens, plan_host,
                        plan_dev, out, visits, stream=None) -> None:
    """Enqueue the coverage-counting debug form of one decode step; `visits`
    is a zeroed device int32 tensor [num_pages * page_size * Hkv]."""
    lib = load_library()
    plan_host = np.ascontiguousarray(plan_host, dtype=np.int32)
    st = lib.hda_decode_coverage(ctypes.byref(params), _ptr(q), _ptr(k_pages), _ptr(v_pages),
                                 _ptr(block_table), _ptr(seq_lens), _i32p(plan_host),
                                 _ptr(plan_dev), plan_host.size, _ptr(out), _ptr(visits),
                                 _stream(stream))
    if st != HDA_OK:
        raise HdaError(st, "hda_decode_coverage")


def hda_decode_check(params: hda_params, n_workgroups: int, stream=None) -> int:
    """Device check bits (HDA_CHECK_*) the last call with this workspace
    recorded; synchronises the stream."""
    flags = ctypes.c_int32(0)
    st = load_library().hda_decode_check(ctypes.byref(params), int(n_workgroups),
                                         ctypes.byref(flags), _stream(stream))
    if st not in (HDA_OK, HDA_ERR_PLAN_MISMATCH):
        raise HdaError(st, "hda_decode_check")
    return flags.value


def hda_workspace_bytes_bound(batch: int, n_workgroups: int, n_q_heads: int, head_dim: int) -> int:
    return load_library().hda_workspace_bytes_bound(int(batch), int(n_workgroups), int(n_q_heads),
                                                    int(head_dim))


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    if hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    return ctypes.c_void_p(int(stream) if stream else 0)


def hda_decode_auto(params: hda_params, q, k_pages, v_pages, block_table, seq_lens,
                    tile_len: int, n_workgroups: int, out, stream=None) -> None:
    """Enqueue one decode step planned on the device from the device lengths."""
    lib = load_library()
    st = lib.hda_decode_auto(ctypes.byref(params), _ptr(q), _ptr(k_pages), _ptr(v_pages),
                             _ptr(block_table), _ptr(seq_lens), int(tile_len), int(n_workgroups),
                             _ptr(out), _stream(stream))
    if st != HDA_OK:
        raise HdaError(st, "hda_decode_auto")


def hda_plan_device(seq_lens, batch: int, tile_len: int, n_workgroups: int, plan, capacity: int,
                    stream=None) -> None:
    """Enqueue the device-side planner writing the hda_plan format into `plan`."""
    lib = load_library()
    st = lib.hda_plan_device(_ptr(seq_lens), int(batch), int(tile_len), int(n_workgroups),
                             _ptr(plan), int(capacity), _stream(stream))
    if st != HDA_OK:
        raise HdaError(st, "hda_plan_device")


def hda_plan_upload(plan, plan_dev, stream=None, plan_len=None) -> None:
    """Enqueue the copy of a host plan (np.int32, first `plan_len` ints) into
    `plan_dev` through store-kernel launch arguments; `plan` may be reused
    once this returns."""
    plan = np.asarray(plan)
    if plan.dtype != np.int32 or not plan.flags.c_contiguous:
        raise TypeError("plan must be a C-contiguous int32 array")
    n = plan.size if plan_len is None else int(plan_len)
    if n > plan.size:
        raise ValueError("plan_len exceeds the host plan")
    if hasattr(plan_dev, "numel") and (plan_dev.element_size() != 4 or plan_dev.numel() < n
                                       or not plan_dev.is_contiguous()):
        raise ValueError("plan_dev must be a contiguous 4-byte tensor of at least plan_len elements")
    lib = load_library()
    st = lib.hda_plan_upload(plan.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), n,
                             _ptr(plan_dev), _stream(stream))
    if st != HDA_OK:
        raise HdaError(st, "hda_plan_upload")


def hda_prefill_rows_per_block(n_q_heads: int, n_kv_heads: int) -> int:
    return load_library().hda_prefill_rows_per_block(int(n_q_heads), int(n_kv_heads))


def hda_prefill_block_rows(q_lens, n_q_heads: int, n_kv_heads: int) -> int:
    """Block size (rows) for a batch: 1, 2, 4, 8 or 16 tiles by the mean query run."""
    ql = _lens(q_lens)
    return load_library().hda_prefill_block_rows(_i32p(ql), len(ql), int(n_q_heads),
                                                 int(n_kv_heads))


def hda_prefill_rows(q_lens, kv_lens, rows_per_block: int):
    """Row blocks of a multi-token batch: (rows int32 [n, 4], row_lens int32 [n])."""
    lib = load_library()
    ql, kl = _lens(q_lens), _lens(kv_lens)
    if len(ql) != len(kl):
        raise ValueError("q_lens and kv_lens differ in length")
    n = ctypes.c_int64(0)
    st = lib.hda_prefill_rows(_i32p(ql), _i32p(kl), len(ql), int(rows_per_block), None, None, 0,
                              ctypes.byref(n))
    if st != HDA_ERR_CAPACITY:
        raise HdaError(st, "hda_prefill_rows")
    rows = np.empty((n.value, 4), dtype=np.int32)
    row_lens = np.empty(n.value, dtype=np.int32)
    st = lib.hda_prefill_rows(_i32p(ql), _i32p(kl), len(ql), int(rows_per_block), _i32p(rows),
                              _i32p(row_lens), n.value, ctypes.byref(n))
    if st != HDA_OK:
        raise HdaError(st, "hda_prefill_rows")
    return rows, row_lens


def hda_prefill_workspace_bytes(plan, n_q_heads: int, n_kv_heads: int, head_dim: int,
                                rows_per_block: int) -> int:
    lib = load_library()
    plan = np.ascontiguousarray(plan, dtype=np.int32)
    return lib.hda_prefill_workspace_bytes(_i32p(plan), plan.size, int(n_q_heads),
                                           int(n_kv_heads), int(head_dim), int(rows_per_block))


def hda_prefill(params: hda_params, q, k_pages, v_pages, block_table, kv_lens, n_q: int,
                rows_host, rows_dev, plan_host, plan_dev, out, stream=None) -> None:
    """Enqueue one multi-token attention step (see include/hda.h)."""
    lib = load_library()
    rows_host = np.ascontiguousarray(rows_host, dtype=np.int32)
    plan_host = np.ascontiguousarray(plan_host, dtype=np.int32)
    st = lib.hda_prefill(ctypes.byref(params), _ptr(q), _ptr(k_pages), _ptr(v_pages),
                         _ptr(block_table), _ptr(kv_lens), int(n_q), _i32p(rows_host),
                         _ptr(rows_dev), _i32p(plan_host), _ptr(plan_dev), plan_host.size,
                         _ptr(out), _stream(stream))
    if st != HDA_OK:
        raise HdaError(st, "hda_prefill")


def hda_router_split_weights(w, w_hi, w_lo, stream=None) -> None:
    """Enqueue the split of fp32 weights w (device) into bf16 hi / lo."""
    n = w.numel() if hasattr(w, "numel") else int(w)
    st = load_library().hda_router_split_weights(_ptr(w), n, _ptr(w_hi), _ptr(w_lo),
                                                 _stream(stream))
    if st != HDA_OK:
        raise HdaError(st, "hda_router_split_weights")


def hda_router_workspace_bytes(tokens: int, experts: int, hidden: int) -> int:
    return load_library().hda_router_workspace_bytes(int(tokens), int(experts), int(hidden))


def hda_router_gemm(x, w_hi, w_lo, tokens: int, experts: int, hidden: int, out, workspace=None,
                    workspace_bytes: int = 0, stream=None) -> None:
    """Enqueue out = x hi^T + (x lo^T)/256 (see include/hda.h)."""
    if workspace is not None and hasattr(workspace, "numel"):
        workspace_bytes = workspace.numel() * workspace.element_size()
    st = load_library().hda_router_gemm(_ptr(x), _ptr(w_hi), _ptr(w_lo), int(tokens),
                                        int(experts), int(hidden), _ptr(out), _ptr(workspace),
                                        int(workspace_bytes), _stream(stream))
    if st != HDA_OK:
        raise HdaError(st, "hda_router_gemm")


def hda_read_probe(buf, n_workgroups: int, sink, stream=None) -> None:
    """Enqueue the streaming-read probe over the device tensor `buf` (see
    include/hda.h); `sink` is a uint32/int32 device tensor of
    n_workgroups * 256 elements."""
    nbytes = buf.numel() * buf.element_size()
    if sink.numel() < int(n_workgroups) * 256:
        raise ValueError("sink smaller than n_workgroups * 256 words")
    st = load_library().hda_read_probe(_ptr(buf), int(nbytes), int(n_workgroups), _ptr(sink),
                                       _stream(stream))
    if st != HDA_OK:
        raise HdaError(st, "hda_read_probe")


class RouterWeights:
    """Device-resident split router weights plus a workspace; convenience for
    tests and the bench."""

    def __init__(self, w, device="cuda:0"):
        import torch
        self.w = torch.as_tensor(w, dtype=torch.float32).to(device).contiguous()
        self.E, self.H = self.w.shape
        self.hi = torch.empty((self.E, self.H), dtype=torch.int16, device=device)
        self.lo = torch.empty_like(self.hi)
        self.device = device
        self._ws = None
        hda_router_split_weights(self.w, self.hi, self.lo)

    def logits(self, x, out=None, stream=None):
        import torch
        T = x.shape[0]
        if out is None:
            out = torch.empty((T, self.E), dtype=torch.float32, device=self.device)
        need = hda_router_workspace_bytes(T, self.E, self.H)
        if need < 0:
            raise HdaError(HDA_ERR_UNSUPPORTED, "hda_router_workspace_bytes")
        if need and (self._ws is None or self._ws.numel() < need):
            self._ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        hda_router_gemm(x, self.hi, self.lo, T, self.E, self.H, out,
                        self._ws if need else None, need, stream)
        return out


def _ptr(x):
    if x is None:
        return None
    if hasattr(x, "data_ptr"):
        return ctypes.c_void_p(x.data_ptr())
    return ctypes.c_void_p(int(x))


class DeviceBatch:
    """Device-resident copy of one generated batch (torch tensors) plus the
    hda_params that describe it.  Convenience for tests and the bench."""

    def __init__(self, tensors, params_kw, device):
        self.t = tensors
        self.kw = params_kw
        self.device = device
        self._ws = None

    @classmethod
    def from_inputs(cls, inp, device="cuda:0", math="bf16"):
        """math "fp8": the native-fp8 product mode, with the V pages stored
        dim-major ([page][Hkv][D][page_size]) on the device."""
        import torch
        w = inp["workload"]
        vp = inp["v_pages"]
        if math == "fp8":
            vp = np.ascontiguousarray(np.swapaxes(vp, 2, 3))
        t = {
            "q": torch.from_numpy(inp["q"].view(np.int16)).to(device),
            "k_pages": torch.from_numpy(inp["k_pages"].view(np.uint8).reshape(-1)).to(device),
            "v_pages": torch.from_numpy(vp.view(np.uint8).reshape(-1)).to(device),
            "block_table": torch.from_numpy(inp["block_table"]).to(device),
            "seq_lens": torch.from_numpy(inp["seq_lens"]).to(device),
        }
        kw = dict(batch=len(inp["seq_lens"]), n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads,
                  head_dim=w.head_dim, page_size=w.page_size,
                  max_pages_per_req=inp["block_table"].shape[1],
                  num_pages=inp["k_pages"].shape[0],
                  kv_dtype=HDA_KV_FP8_E4M3 if w.kv_dtype == "fp8" else HDA_KV_BF16,
                  sm_scale=float(inp["sm_scale"]), k_scale=float(inp["k_scale"]),
                  v_scale=float(inp["v_scale"]), prologue=0,
                  math=HDA_MATH_FP8 if math == "fp8" else HDA_MATH_BF16,
                  v_layout=HDA_V_DIM_MAJOR if math == "fp8" else HDA_V_TOKEN_MAJOR)
        if w.prologue:
            for k in ("q_norm_w", "k_norm_w", "k_new", "v_new"):
                t[k] = torch.from_numpy(inp[k].view(np.int16)).to(device)
            kw.update(prologue=1, rms_eps=float(inp["rms_eps"]), rope_theta=float(inp["rope_theta"]))
        mode = inp.get("scale_mode", "tensor")
        kw["scale_mode"] = SCALE_MODES[mode]
        if mode != "tensor":
            for k in ("k_scales", "v_scales"):
                t[k] = torch.from_numpy(np.ascontiguousarray(inp[k], dtype=np.float32)).to(device)
        return cls(t, kw, device)

    def v_pages_token_major(self, shape):
        """The device V pool read back as numpy [NP, Hkv, ps, D] in the
        token-major order, whatever the device layout (raw element bits)."""
        dt = np.uint8 if self.kw["kv_dtype"] == HDA_KV_FP8_E4M3 else np.uint16
        raw = self.t["v_pages"].cpu().numpy().view(dt)
        if self.kw.get("v_layout") == HDA_V_DIM_MAJOR:
            NP, Hkv, ps, D = shape
            return np.swapaxes(raw.reshape(NP, Hkv, D, ps), 2, 3)
        return raw.reshape(shape)

    def workspace(self, nbytes):
        import torch
        if self._ws is None or self._ws.numel() < nbytes:
            self._ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
        return self._ws

    def params(self, plan, workspace=None, need=None):
        p = hda_params(**self.kw)
        t = self.t
        if "k_scales" in t:
            p.k_scales = t["k_scales"].data_ptr()
            p.v_scales = t["v_scales"].data_ptr()
        if self.kw.get("prologue"):
            p.q_norm_w = t["q_norm_w"].data_ptr()
            p.k_norm_w = t["k_norm_w"].data_ptr()
            p.k_new = t["k_new"].data_ptr()
            p.v_new = t["v_new"].data_ptr()
        if need is None:
            need = hda_workspace_bytes(plan, self.kw["n_q_heads"], self.kw["n_kv_heads"],
                                       self.kw["head_dim"])
        ws = workspace if workspace is not None else self.workspace(need)
        p.workspace = ws.data_ptr()
        p.workspace_bytes = ws.numel() * ws.element_size()
        return p

    def params_auto(self, tile_len, n_workgroups, workspace=None):
        p = self.params(None, workspace=workspace, need=hda_workspace_bytes_bound(
            self.kw["batch"], n_workgroups, self.kw["n_q_heads"], self.kw["head_dim"]))
        return p

    def decode_auto(self, tile_len, n_workgroups, out=None, stream=None, k_pages=None,
                    v_pages=None):
        import torch
        t = self.t
        if out is None:
            out = torch.empty((self.kw["batch"], self.kw["n_q_heads"], self.kw["head_dim"]),
                              dtype=torch.float32, device=self.device)
        p = self.params_auto(tile_len, n_workgroups)
        hda_decode_auto(p, t["q"], t["k_pages"] if k_pages is None else k_pages,
                        t["v_pages"] if v_pages is None else v_pages, t["block_table"],
                        t["seq_lens"], tile_len, n_workgroups, out, stream)
        return out

    def prefill_plan(self, q_lens, tile_len=None, n_workgroups=None, tiles=None):
        """(rows, plan) for this batch's query rows (row blocks through the
        decode planner); blocks of `tiles` x the column-filling size (default:
        hda_prefill_block_rows); default launch shape from launch_config."""
        kv = self.t["seq_lens"].cpu().numpy()
        hq, hk = self.kw["n_q_heads"], self.kw["n_kv_heads"]
        qb = (hda_prefill_block_rows(q_lens, hq, hk) if tiles is None
              else tiles * hda_prefill_rows_per_block(hq, hk))
        rows, row_lens = hda_prefill_rows(q_lens, kv, qb)
        tl, W = launch_config(row_lens, self.kw["n_kv_heads"])
        return rows, hda_plan(row_lens, tile_len or tl, n_workgroups or W)

    def prefill_params(self, plan, rows_per_block=None):
        p = hda_params(**self.kw)
        t = self.t
        if "k_scales" in t:
            p.k_scales = t["k_scales"].data_ptr()
            p.v_scales = t["v_scales"].data_ptr()
        if rows_per_block is None:      # enough for any block
            rows_per_block = HDA_PREFILL_MAX_TILES * hda_prefill_rows_per_block(
                self.kw["n_q_heads"], self.kw["n_kv_heads"])
        need = hda_prefill_workspace_bytes(plan, self.kw["n_q_heads"], self.kw["n_kv_heads"],
                                           self.kw["head_dim"], rows_per_block)
        ws = self.workspace(need)
        p.workspace = ws.data_ptr()
        p.workspace_bytes = ws.numel()
        return p

    def prefill(self, rows, plan, out=None, stream=None, rows_dev=None, plan_dev=None):
        import torch
        rows = np.ascontiguousarray(rows, dtype=np.int32)
        plan = np.ascontiguousarray(plan, dtype=np.int32)
        t = self.t
        n_q = t["q"].shape[0]
        if out is None:
            out = torch.empty((n_q, self.kw["n_q_heads"], self.kw["head_dim"]),
                              dtype=torch.float32, device=self.device)
        if rows_dev is None:
            rows_dev = torch.from_numpy(rows.reshape(-1)).to(self.device)
        if plan_dev is None:
            plan_dev = torch.from_numpy(plan).to(self.device)
        p = self.prefill_params(plan)
        hda_prefill(p, t["q"], t["k_pages"], t["v_pages"], t["block_table"], t["seq_lens"], n_q,
                    rows, rows_dev, plan, plan_dev, out, stream)
        return out

    def decode(self, plan, out=None, plan_dev=None, stream=None, k_pages=None, v_pages=None,
               block_table=None, seq_lens=None, upload="copy"):
        """One decode step.  upload: "copy" (the plan copied to a device
        tensor, or the given plan_dev), or "bench" -- the plan in the tile
        kernel's launch arguments when it fits, else hda_plan_upload into a
        device buffer: the path bench.py times (plan_to_device)."""
        import torch
        plan = np.ascontiguousarray(plan, dtype=np.int32)
        t = self.t
        if out is None:
            out = torch.empty((self.kw["batch"], self.kw["n_q_heads"], self.kw["head_dim"]),
                              dtype=torch.float32, device=self.device)
        if upload == "bench":
            if plan_dev is None:
                plan_dev = torch.empty(plan.size, dtype=torch.int32, device=self.device)
            plan_dev = plan_to_device(plan, plan.size, plan_dev, stream)
        elif plan_dev is None:
            plan_dev = torch.from_numpy(plan).to(self.device)
        p = self.params(plan)
        self.last_params = p
        hda_decode(p, t["q"], t["k_pages"] if k_pages is None else k_pages,
                   t["v_pages"] if v_pages is None else v_pages,
                   t["block_table"] if block_table is None else block_table,
                   t["seq_lens"] if seq_lens is None else seq_lens, plan, plan_dev, out, stream)
        return out

    def check(self, plan, stream=None):
        """HDA_CHECK_* bits the last decode with this batch's workspace recorded."""
        return hda_decode_check(self.last_params, int(np.asarray(plan)[3]), stream)

    def coverage(self, plan, seq_lens=None, block_table=None):
        """(out, visits) of the coverage-counting debug step: visits int32
        [num_pages, page_size, Hkv] on the device."""
        import torch
        plan = np.ascontiguousarray(plan, dtype=np.int32)
        t = self.t
        kw = self.kw
        out = torch.empty((kw["batch"], kw["n_q_heads"], kw["head_dim"]), dtype=torch.float32,
                          device=self.device)
        visits = torch.zeros((kw["num_pages"], kw["page_size"], kw["n_kv_heads"]),
                             dtype=torch.int32, device=self.device)
        p = self.params(plan)
        hda_decode_coverage(p, t["q"], t["k_pages"], t["v_pages"],
                            t["block_table"] if block_table is None else block_table,
                            t["seq_lens"] if seq_lens is None else seq_lens, plan,
                            torch.from_numpy(plan).to(self.device), out, visits)
        return out, visits


def plan_to_device(plan_host, plan_len: int, plan_dev, stream=None):
    """The per-step plan upload bench.py times: None when the plan fits the
    tile kernel's launch arguments (hda_decode then carries it there), else
    the plan stored into plan_dev by hda_plan_upload, returning plan_dev."""
    if plan_len <= HDA_PLAN_ARG_INTS:
        return None
    hda_plan_upload(plan_host, plan_dev, stream, plan_len=plan_len)
    return plan_dev


def launch_config(seq_lens, n_kv_heads: int, n_cu: int = 256, wg_per_cu: int = 2,
                  tile_len: int = 128):
    """Default (tile_len, n_workgroups) for a step (hda_launch_config: the
    fewest tiles on the busiest compute unit, up to `wg_per_cu` workgroups
    per unit, then the fewest partial slots)."""
    lens = _lens(seq_lens)
    W = ctypes.c_int32(0)
    st = load_library().hda_launch_config(_i32p(lens), len(lens), int(n_kv_heads), int(n_cu),
                                          int(wg_per_cu), int(tile_len), ctypes.byref(W))
    if st != HDA_OK:
        raise HdaError(st, "hda_launch_config")
    return tile_len, W.value

#!/usr/bin/env python3
"""Decode-attention step benchmark on one MI355X.

A step is one pass of the whole hot path over one batch: the host planner
(hda_plan) rebuilds the tile plan from the current lengths, the plan goes to
the device inside the tile kernel's launch arguments (plans longer than
HDA_PLAN_ARG_INTS ints through hda_plan_upload; `--upload copy` for an async
copy from pinned memory), and hda_decode runs the attention kernel (tile
loads, QK, online softmax, PV, log-sum-exp merge) on the torch stream.  Inputs are resident in HBM before timing starts.

Default workload: the 1 x 131072 + 31 x 4096 extreme mix (bf16 cache, 64 q /
8 kv heads, head dim 128, page 64, random page placement).  The KV pools are
held in several copies and steps rotate over them so that no step finds the
previous step's bytes in the 256 MB last-level cache.

Prints one JSON line: value = KV bytes read per second (GB/s), plus the
kernel's roofline position (HIP-event durations on the launch stream), the
load-balance gain over static split plans, and the fp64 oracle timed on a
bounded sample of the same workload on the host cores.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E spec
MFMA_BF16_PEAK_TFLOPS = 2500.0 # MI355X dense bf16
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SRC = os.path.join(ROOT, "load_balanced_split_step_amd", "csrc", "hda_decode.hip")
METRIC = "decode-attn µs/step + KV GB/s (% HBM peak), 1×128K+31×4K mix, 1 GPU"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="extreme")
    ap.add_argument("--kv-scale", choices=["tensor", "head", "page"], default=None,
                    help="override the workload's fp8 scale granularity")
    ap.add_argument("--math", choices=["bf16", "fp8"], default="bf16",
                    help="product arithmetic: bf16 (cache widened to bf16) or fp8 (native fp8 "
                         "MFMA operands, V pages dim-major; fp8 cache only)")
    ap.add_argument("--tiles", choices=["auto", "1", "2", "4", "8", "16"], default="auto",
                    help="multi-token workloads: row blocks of this many tiles of 16/group rows "
                         "(above 1: K/V chunks shared through LDS); auto: by the mean query run")
    ap.add_argument("--tile-len", type=int, default=None)
    ap.add_argument("--workgroups", type=int, default=None)
    ap.add_argument("--copies", type=int, default=4, help="KV pool copies rotated over")
    ap.add_argument("--upload", choices=["args", "kernel", "copy"], default="args",
                    help="plan upload: in the tile kernel's launch arguments (plans up to "
                         "HDA_PLAN_ARG_INTS ints, else as 'kernel'), in a store kernel's "
                         "launch arguments (hda_plan_upload), or an async copy from pinned memory")
    ap.add_argument("--no-static", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 1 GiB device-to-device copy (counter calibration)")
    ap.add_argument("--no-read-probe", action="store_true",
                    help="skip the streaming-read probe (a pure read of the tile kernel's "
                         "algorithmic bytes: the measured read ceiling)")
    return ap.parse_args()


def read_probe(nbytes, reps=10):
    """The measured read ceiling for a launch that must read `nbytes`:
    hda_read_probe (each wave streams its own contiguous region, 16-byte
    non-temporal loads) over that many bytes, best of a few launch sizes,
    timed with events on the current stream."""
    import torch
    import load_balanced_split_step_amd.hda as hda
    nbytes = (int(nbytes) + 15) // 16 * 16
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda:0")
    best = None
    for wgs in (256, 512, 1024, 2048):
        sink = torch.empty(wgs * 256, dtype=torch.int32, device="cuda:0")
        hda.hda_read_probe(buf, wgs, sink)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            hda.hda_read_probe(buf, wgs, sink)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        gbs = nbytes / (us * 1e-6) / 1e9
        if best is None or gbs > best["gbs"]:
            best = {"bytes": nbytes, "n_workgroups": wgs, "us": round(us, 2), "gbs": round(gbs, 1),
                    "kernel": "hda_read_probe_kernel"}
    del buf
    return best


def single_stream_gbs(nbytes=64 << 20, reps=5):
    """Read rate of one 4-wave workgroup alone on the GPU (hda_read_probe with
    one workgroup): what a static split's longest chunk streams at."""
    import torch
    import load_balanced_split_step_amd.hda as hda
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda:0")
    sink = torch.empty(256, dtype=torch.int32, device="cuda:0")
    hda.hda_read_probe(buf, 1, sink)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        hda.hda_read_probe(buf, 1, sink)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    del buf
    return nbytes / (us * 1e-6) / 1e9


def algorithmic_bytes(inp, plan_len):
    """Bytes one launch must move: every cached K/V row of every kv head,
    q, the output, the block-table entries in use, lengths and plan."""
    from load_balanced_split_step_amd.workloads import kv_bytes
    w = inp["workload"]
    B = len(inp["seq_lens"])
    pages_used = int(sum(-(-int(L) // w.page_size) for L in inp["seq_lens"]))
    return (kv_bytes(inp) + B * w.n_q_heads * w.head_dim * 2 + B * w.n_q_heads * w.head_dim * 4
            + pages_used * 4 + B * 4 + plan_len * 4)


def traffic_from_profiles(workload):
    """Measured HBM bytes per launch from the committed counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(PROFILES, f"hda_decode_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    sha = hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()
    if rec.get("kernel_source_sha256") != sha:
        return None
    return rec.get("bytes_per_launch")


def time_plan_kernel(dev, plan, copies, steps, warmup):
    """Kernel-only durations (ms) of hda_decode for a fixed plan."""
    import numpy as np
    import torch
    pd = torch.from_numpy(np.ascontiguousarray(plan)).to(dev.device)
    out = torch.empty((dev.kw["batch"], dev.kw["n_q_heads"], dev.kw["head_dim"]),
                      dtype=torch.float32, device=dev.device)
    evs = []
    for s in range(warmup + steps):
        kp, vp = copies[s % len(copies)]
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        dev.decode(plan, out=out, plan_dev=pd, k_pages=kp, v_pages=vp)
        e1.record()
        if s >= warmup:
            evs.append((e0, e1))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def host_info():
    """The host the oracle runs on: cores this process may use, the OS's
    CPU count, the CPU model, and the BLAS threads numpy's matrix products
    use (the oracle's parallelism)."""
    from threadpoolctl import threadpool_info
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:
        aff = os.cpu_count()
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"affinity_cores": int(aff), "os_cpu_count": os.cpu_count(), "cpu_model": model,
            "blas_threads": int(blas)}


def cpu_baseline(inp, budget_s, one_thread=False):
    """The fp64 oracle, as it stands, on a bounded sample of the workload:
    whole requests, shortest first, cycling over the batch until the time
    budget is spent.  Rate = KV bytes of the requests done / seconds.  With
    one_thread, BLAS is held to one thread."""
    import contextlib
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_limits
    w = inp["workload"]
    order = np.argsort(inp["seq_lens"], kind="stable")
    q64 = oracle.bf16_to_f64(inp["q"])
    done, toks = [], 0
    seq = order.tolist() * 64
    limit = threadpool_limits(limits=1) if one_thread else contextlib.nullcontext()
    with limit:
        info = host_info()
        t0 = time.perf_counter()
        toks, done = _oracle_passes(inp, q64, seq, budget_s, t0)
    secs = time.perf_counter() - t0
    elem = 1 if w.kv_dtype == "fp8" else 2
    kvb = toks * w.n_kv_heads * w.head_dim * 2 * elem
    threads = info["blas_threads"]
    return {"value": round(kvb / secs / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", **{k: v for k, v in info.items() if k != "blas_threads"},
            "sample": f"{len(done)} request passes over the {len(inp['seq_lens'])}-request "
                      f"batch, shortest first ({toks} KV tokens) in {secs:.1f} s; "
                      f"numpy fp64, BLAS threads {threads} (cores = the BLAS threads used)"}


def _oracle_passes(inp, q64, seq, budget_s, t0):
    import oracle
    w = inp["workload"]
    done, toks = [], 0
    for b in seq:
        sub = [b]
        oracle.attention_reference(q64[sub], inp["k_pages"], inp["v_pages"],
                                   inp["block_table"][sub], inp["seq_lens"][sub], w.kv_dtype,
                                   float(inp["sm_scale"]), float(inp["k_scale"]),
                                   float(inp["v_scale"]), scale_mode=inp["scale_mode"],
                                   k_scales=inp["k_scales"], v_scales=inp["v_scales"])
        done.append(b)
        toks += int(inp["seq_lens"][b])
        if time.perf_counter() - t0 >= budget_s:
            break
    return toks, done


def cpu_baseline_prefill(inp, budget_s):
    """The fp64 prefill oracle, as it stands, on a bounded sample: whole
    requests, shortest cache first, until the time budget is spent.  Rate =
    KV bytes each query row reads (its causal prefix) per second."""
    import numpy as np
    import oracle
    w = inp["workload"]
    order = np.argsort(inp["seq_lens"], kind="stable")
    off = oracle.q_offsets(inp["q_lens"])
    elem = 1 if w.kv_dtype == "fp8" else 2
    done, kvb, t0 = 0, 0, time.perf_counter()
    for b in order.tolist() * 8:
        sub = dict(block_table=inp["block_table"][[b]], seq_lens=inp["seq_lens"][[b]],
                   q_lens=inp["q_lens"][[b]])
        oracle.prefill_reference(oracle.bf16_to_f64(inp["q"][off[b]:off[b + 1]]), inp["k_pages"],
                                 inp["v_pages"], sub["block_table"], sub["seq_lens"],
                                 sub["q_lens"], w.kv_dtype, float(inp["sm_scale"]),
                                 float(inp["k_scale"]), float(inp["v_scale"]))
        L, n = int(inp["seq_lens"][b]), int(inp["q_lens"][b])
        kvb += sum(L - n + r + 1 for r in range(n)) * w.n_kv_heads * w.head_dim * 2 * elem
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    secs = time.perf_counter() - t0
    info = host_info()
    threads = info.pop("blas_threads")
    return {"value": round(kvb / secs / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", **info,
            "sample": f"{done} request passes (shortest caches first) in {secs:.1f} s; "
                      f"numpy fp64, BLAS threads {threads} (cores = the BLAS threads used)"}


def bench_prefill(args, w, inp):
    """Multi-token step: row blocks and plan on the host from the current
    lengths, both uploaded in one hda_plan_upload call (rows, then the plan,
    in one device buffer; `--upload copy`: two async copies from pinned
    memory), hda_prefill."""
    import numpy as np
    import torch
    import load_balanced_split_step_amd.hda as hda
    lens, qlens = inp["seq_lens"], inp["q_lens"]
    dev = hda.DeviceBatch.from_inputs(inp, device="cuda:0")
    copies = [(dev.t["k_pages"], dev.t["v_pages"])]
    for _ in range(max(0, args.copies - 1)):
        copies.append((dev.t["k_pages"].clone(), dev.t["v_pages"].clone()))
    unit = hda.hda_prefill_rows_per_block(w.n_q_heads, w.n_kv_heads)
    def block_rows():
        if args.tiles == "auto":
            return hda.hda_prefill_block_rows(qlens, w.n_q_heads, w.n_kv_heads)
        return int(args.tiles) * unit

    qb = block_rows()
    tiles = qb // unit
    rows, row_lens = hda.hda_prefill_rows(qlens, lens, qb)
    tl, W = hda.launch_config(row_lens, w.n_kv_heads)
    tl = args.tile_len or tl
    W = args.workgroups or W
    R = len(rows)
    cap = hda.hda_plan_capacity(R, W)
    NB = 3
    pin_plan = [torch.empty(cap, dtype=torch.int32).pin_memory() for _ in range(NB)]
    pin_rows = [torch.empty(4 * R, dtype=torch.int32).pin_memory() for _ in range(NB)]
    d_plan = [torch.empty(cap, dtype=torch.int32, device="cuda:0") for _ in range(NB)]
    d_rows = [torch.empty(4 * R, dtype=torch.int32, device="cuda:0") for _ in range(NB)]
    # one upload of [rows | plan]: 4R ints keep the plan 16-byte aligned
    host_both = np.empty(4 * R + cap, dtype=np.int32)
    d_both = [torch.empty(4 * R + cap, dtype=torch.int32, device="cuda:0") for _ in range(NB)]
    n_q = int(qlens.sum())
    out = torch.empty((n_q, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream()
    done_ev = [torch.cuda.Event() for _ in range(NB)]
    used = [False] * NB
    params = dev.prefill_params(hda.hda_plan(row_lens, tl, W), rows_per_block=qb)

    def step(s, events=None):
        j = s % NB
        if used[j]:
            done_ev[j].synchronize()
        r, rl = hda.hda_prefill_rows(qlens, lens, block_rows())          # row blocks
        if args.upload == "copy":
            pin_rows[j].numpy()[:] = r.reshape(-1)
            n = hda.hda_plan_into(rl, tl, W, pin_plan[j].numpy())       # the decode planner
            d_rows[j].copy_(pin_rows[j], non_blocking=True)
            d_plan[j][:n].copy_(pin_plan[j][:n], non_blocking=True)
            done_ev[j].record(stream)
            used[j] = True
            h_rows, h_plan = pin_rows[j].numpy(), pin_plan[j].numpy()[:n]
            dr, dp = d_rows[j], d_plan[j]
        else:
            host_both[:4 * R] = r.reshape(-1)
            n = hda.hda_plan_into(rl, tl, W, host_both[4 * R:])         # the decode planner
            hda.hda_plan_upload(host_both, d_both[j], stream, plan_len=4 * R + n)
            h_rows, h_plan = host_both[:4 * R], host_both[4 * R:4 * R + n]
            dr, dp = d_both[j][:4 * R], d_both[j][4 * R:]
        kp, vp = copies[s % len(copies)]
        if events is not None:
            events[0].record(stream)
            params.split_event = events[1].cuda_event
        else:
            params.split_event = None
        hda.hda_prefill(params, dev.t["q"], kp, vp, dev.t["block_table"], dev.t["seq_lens"], n_q,
                        h_rows.reshape(R, 4), dr, h_plan, dp, out, stream)
        if events is not None:
            events[2].record(stream)
        return n

    for s in range(args.warmup):
        plan_len = step(s)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        plan_len = step(args.warmup + s)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    n_prof = max(10, min(args.steps, 50))
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(n_prof)]
    for e in evs:
        for x in e:
            x.record(stream)
    torch.cuda.synchronize()
    for s in range(n_prof):
        step(s, evs[s])
    torch.cuda.synchronize()
    kmean = sum(a.elapsed_time(b) for a, b, _ in evs) / n_prof
    dmean = sum(a.elapsed_time(c) for a, _, c in evs) / n_prof
    elem = 1 if w.kv_dtype == "fp8" else 2
    per_tok = w.n_kv_heads * w.head_dim * 2 * elem
    unique_kv = int(lens.astype(np.int64).sum()) * per_tok
    # algorithmic bytes: every request's cache read once, plus q, out and the
    # tables.  This design reads each row block's causal prefix (reread_kv,
    # reported as kv_read_factor): the cost of its block size, not the method's.
    reread_kv = int(np.asarray(row_lens, np.int64).sum()) * per_tok
    algo = unique_kv + n_q * w.n_q_heads * w.head_dim * (2 + 4) + R * 16 + plan_len * 4
    achieved = algo / (kmean * 1e-3) / 1e9
    # matrix-core work: QK and PV, 2 flops per multiply-add, over each row's
    # causal extent (position + 1 cached tokens)
    extents = sum(int(k) - int(q) + r + 1 for k, q in zip(lens, qlens) for r in range(int(q)))
    flops = 4 * w.head_dim * w.n_q_heads * extents
    tflops = flops / (kmean * 1e-3) / 1e12
    # roofline: HBM below the bf16 ridge point (peak flops / peak bytes)
    mfma_bound = flops / algo > MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    log(f"prefill step {ms_per_step * 1e3:.1f} us wall, kernels {dmean * 1e3:.1f} us, "
        f"tile kernel {kmean * 1e3:.1f} us; {R} row blocks of <= {qb} rows "
        f"({tiles} tile{'s' if tiles > 1 else ''} of {unit}"
        f"{', K/V chunks shared through LDS' if tiles > 1 else ''}), "
        f"KV read {reread_kv / unique_kv:.2f}x the cache; {tflops:.0f} TFLOP/s "
        f"({flops / algo:.0f} flop/B)")
    kernel_name = ("hda_prefill_shared_kernel (HIP events on its stream)" if tiles > 1 else
                   "hda_decode_kernel, multi-token rows (HIP events on its stream)")
    if mfma_bound:
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                "algorithmic_flops": flops, "kernel": kernel_name}
    else:
        roof = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                "algorithmic_bytes": algo, "kernel": kernel_name}
    res = {
        "metric": "multi-token attention: query rows/s (row blocks through the decode planner), 1 GPU",
        "value": round(n_q / (ms_per_step * 1e-3), 1),
        "unit": "query rows/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if w.kv_dtype == "bf16" else "fp8",
        "data": "synthetic",
        "plan_upload": "copy" if args.upload == "copy" else "kernel (rows and plan, one launch)",
        "config": {"workload": f"{args.workload}: {len(lens)} requests, {n_q} query rows over "
                               f"{int(lens.sum())} cached tokens",
                   "batch": int(len(lens)), "query_rows": n_q, "kv_tokens": int(lens.sum()),
                   "q_heads": w.n_q_heads, "kv_heads": w.n_kv_heads, "head_dim": w.head_dim,
                   "page_size": w.page_size, "kv_dtype": w.kv_dtype, "rows_per_block": qb,
                   "tiles_per_block": tiles, "shared_chunks": tiles > 1,
                   "row_blocks": R, "tile_len": tl, "n_workgroups": W},
        "us_per_step": {"wall": round(ms_per_step * 1e3, 2), "kernels_mean": round(dmean * 1e3, 2),
                        "tile_kernel_mean": round(kmean * 1e3, 2)},
        "kv_gbs_unique": round(unique_kv / (dmean * 1e-3) / 1e9, 2),
        "kv_read_factor": round(reread_kv / unique_kv, 3),
        "roofline": roof,
        "matrix_core": {"algorithmic_flops": flops, "tflops": round(tflops, 2),
                        "peak_tflops": MFMA_BF16_PEAK_TFLOPS,
                        "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                        "flop_per_byte": round(flops / algo, 1)},
    }
    if not args.no_read_probe:
        res["read_probe"] = read_probe(algo)
        log(f"read probe: {res['read_probe']['gbs']:.0f} GB/s reading the same "
            f"{algo / 1e9:.2f} GB; the tile kernel moves its bytes at "
            f"{achieved / res['read_probe']['gbs']:.1%} of that rate")
    if not args.no_cpu:
        log("timing the fp64 prefill oracle on a bounded sample")
        res["cpu_baseline"] = cpu_baseline_prefill(inp, args.cpu_seconds)
    print(json.dumps(res), flush=True)




def bench_router(args):
    """Router GEMM sweep over token counts (decode batch to prefill): the
    fused split kernel (two bf16 MFMA products per K step, fp32 accumulate),
    device time per call from a replayed HIP graph of 10 calls (HIP events
    on the replay stream), its roofline position, and torch's fp32 GEMM on
    the same data, timed the same way, as context."""
    import numpy as np
    import torch
    import load_balanced_split_step_amd.hda as hda
    from load_balanced_split_step_amd.workloads import ROUTER_CONFIGS, make_router_inputs
    w = ROUTER_CONFIGS["router"]
    E, H = w.experts, w.hidden
    Ts = [1, 4, 8, 16, 64, 256, 1024, 4096, 16384]
    big = make_router_inputs(w, tokens=max(Ts))
    rw = hda.RouterWeights(big["w"])
    wf = torch.from_numpy(big["w"]).cuda()
    x_all = torch.from_numpy(big["x"].view(np.int16)).cuda()
    stream = torch.cuda.current_stream()
    sweep = []
    for T in Ts:
        x = x_all[:T].contiguous()
        xf = x.view(torch.bfloat16).float()
        out = torch.empty((T, E), dtype=torch.float32, device="cuda:0")

        def run_ours():
            rw.logits(x, out=out, stream=torch.cuda.current_stream())

        def run_f32():
            torch.matmul(xf, wf.T)

        res = {}
        for name, fn in (("ours", run_ours), ("torch_fp32", run_f32)):
            for _ in range(args.warmup):
                fn()
            torch.cuda.synchronize()
            # device time per call: a HIP graph of `calls` back-to-back calls,
            # replayed, so that host launch costs do not enter
            calls = 10
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(calls):
                    fn()
            g.replay()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(max(1, args.steps // 2)):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            res[name] = e0.elapsed_time(e1) * 1e3 / (calls * max(1, args.steps // 2))
            del g
        flops = 4.0 * T * H * E                                          # two products
        ws = hda.hda_router_workspace_bytes(T, E, H)
        nbytes = T * H * 2 + E * H * 4 + T * E * 4 + 2 * ws
        inten = flops / nbytes
        bound = "mfma" if inten > MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9) else "hbm"
        if bound == "mfma":
            ach, peak, unit = flops / (res["ours"] * 1e-6) / 1e12, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s"
        else:
            ach, peak, unit = nbytes / (res["ours"] * 1e-6) / 1e9, HBM_PEAK_GBS, "GB/s"
        row = {"tokens": T, "us": round(res["ours"], 2), "torch_fp32_us": round(res["torch_fp32"], 2),
               "speedup_vs_fp32": round(res["torch_fp32"] / res["ours"], 2),
               "tflops": round(flops / (res["ours"] * 1e-6) / 1e12, 1), "bound": bound,
               "achieved": round(ach, 1), "peak": peak, "unit": unit, "frac": round(ach / peak, 4),
               "workspace_bytes": ws}
        sweep.append(row)
        log(f"router T={T}: {res['ours']:.1f} us ({row['tflops']} TFLOP/s, {bound} {row['frac']:.3f}), "
            f"torch fp32 {res['torch_fp32']:.1f} us")
    head = sweep[-1]
    res = {
        "metric": "router GEMM (fp32 weights as bf16 hi + residual/256, fused): TFLOP/s at 16384 tokens, 1 GPU",
        "value": head["tflops"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(head["us"] * 1e-3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"router logits: hidden {H}, {E} experts, tokens {Ts}",
                   "hidden": H, "experts": E},
        "roofline": {"bound": head["bound"], "achieved": head["achieved"], "peak": head["peak"],
                     "unit": head["unit"], "frac": head["frac"], "traffic": None,
                     "kernel": "hda_router_gemm_lds_kernel at 16384 tokens (graph replay, HIP events)"},
        "sweep": sweep,
    }
    if not args.no_cpu:
        # the fp64 oracle on a bounded sample: exact split products of
        # 1024-token batches, repeated until the time budget is spent
        import oracle
        log("timing the fp64 router oracle on a bounded sample")
        x = big["x"][:1024]
        hi, lo = oracle.split_router_weights(big["w"])
        n, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < args.cpu_seconds:
            oracle.router_split_reference(x, hi, lo)
            n += 1
        secs = time.perf_counter() - t0
        info = host_info()
        threads = info.pop("blas_threads")
        res["cpu_baseline"] = {"value": round(n * 4.0 * 1024 * H * E / secs / 1e12, 4),
                               "unit": "TFLOP/s", "cores": threads, "kind": "oracle", **info,
                               "sample": f"{n} exact split products of 1024 tokens in {secs:.1f} s; "
                                         f"numpy fp64, BLAS threads {threads} (cores = the BLAS "
                                         f"threads used)"}
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py times one GPU: --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch
    import load_balanced_split_step_amd.hda as hda
    from load_balanced_split_step_amd.workloads import CONFIGS, make_inputs, kv_bytes

    if args.workload == "router":
        bench_router(args)
        return
    w = CONFIGS[args.workload]
    if args.kv_scale:
        w = w.with_(kv_scale=args.kv_scale)
    t = time.time()
    inp = make_inputs(w)
    log(f"generated {args.workload} inputs in {time.time() - t:.1f}s")
    if w.prefill:
        bench_prefill(args, w, inp)
        return
    lens = inp["seq_lens"]
    dev = hda.DeviceBatch.from_inputs(inp, device="cuda:0", math=args.math)
    copies = [(dev.t["k_pages"], dev.t["v_pages"])]
    for _ in range(max(0, args.copies - 1)):
        copies.append((dev.t["k_pages"].clone(), dev.t["v_pages"].clone()))
    torch.cuda.synchronize()

    tl, W = hda.launch_config(lens, w.n_kv_heads)
    tl = args.tile_len or tl
    W = args.workgroups or W
    cap = hda.hda_plan_capacity(len(lens), W)
    NB = 3                                     # pinned plan buffers in rotation
    pinned = [torch.empty(cap, dtype=torch.int32).pin_memory() for _ in range(NB)]
    plan_dev = [torch.empty(cap, dtype=torch.int32, device="cuda:0") for _ in range(NB)]
    out = torch.empty((len(lens), w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream()
    kv = kv_bytes(inp)
    done_ev = [torch.cuda.Event() for _ in range(NB)]
    used = [False] * NB
    # hda_params does not change between steps of one batch shape
    n0 = hda.hda_plan_into(lens, tl, W, pinned[0].numpy())
    params = dev.params(pinned[0].numpy()[:n0])

    def step(s, events=None):
        j = s % NB
        if used[j]:
            done_ev[j].synchronize()           # the copy that last read pinned[j] is done
        host = pinned[j].numpy()
        n = hda.hda_plan_into(lens, tl, W, host)                  # a1: plan from current lengths
        # a2: upload on the same stream; launch arguments are copied when the
        # launch is enqueued, so only the async copy holds on to pinned[j]
        dplan = plan_dev[j]
        if args.upload == "args":
            # in hda_decode's launch arguments, or hda_plan_upload when longer
            dplan = hda.plan_to_device(host, n, plan_dev[j], stream)
        elif args.upload == "kernel":
            hda.hda_plan_upload(host, plan_dev[j], stream, plan_len=n)
        else:
            plan_dev[j][:n].copy_(pinned[j][:n], non_blocking=True)
            done_ev[j].record(stream)
            used[j] = True
        kp, vp = copies[s % len(copies)]
        if events is not None:
            events[0].record(stream)
            params.split_event = events[1].cuda_event   # recorded between tile and merge kernels
        else:
            params.split_event = None
        hda.hda_decode(params, dev.t["q"], kp, vp, dev.t["block_table"], dev.t["seq_lens"],
                       host[:n], dplan, out, stream)                     # a3..a9
        if events is not None:
            events[2].record(stream)
        return n

    for s in range(args.warmup):
        plan_len = step(s)
    torch.cuda.synchronize()
    # timed region: exactly `steps` steps, nothing else enqueued
    t0 = time.perf_counter()
    for s in range(args.steps):
        plan_len = step(args.warmup + s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    # a1 and a2 apart, outside the timed region: the host planner (C++) and
    # the plan's upload (HIP events around the copy on the launch stream)
    host0 = pinned[0].numpy()
    t0 = time.perf_counter()
    for _ in range(200):
        n_plan = hda.hda_plan_into(lens, tl, W, host0)
    host_plan_us = (time.perf_counter() - t0) * 1e6 / 200
    torch.cuda.synchronize()
    u0, u1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    u0.record(stream)
    upload_mode = ("args" if args.upload == "args" and n_plan <= hda.HDA_PLAN_ARG_INTS
                   else "kernel" if args.upload != "copy" else "copy")
    for _ in range(50):         # in "args" mode the plan rides in the tile launch: 0 here
        if upload_mode == "kernel":
            hda.hda_plan_upload(host0, plan_dev[0], stream, plan_len=n_plan)
        elif upload_mode == "copy":
            plan_dev[0][:n_plan].copy_(pinned[0][:n_plan], non_blocking=True)
    u1.record(stream)
    torch.cuda.synchronize()
    upload_us = u0.elapsed_time(u1) * 1e3 / 50
    log(f"host plan {host_plan_us:.1f} us, plan upload {upload_us:.1f} us ({n_plan} ints)")

    # separate pass with HIP events on the launch stream for kernel durations
    n_prof = max(10, min(args.steps, 50))
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(n_prof)]
    for e in evs:                    # create the underlying HIP events before use
        for x in e:
            x.record(stream)
    torch.cuda.synchronize()
    for s in range(n_prof):
        step(s, evs[s])
    torch.cuda.synchronize()
    tile_ms = sorted(a.elapsed_time(b) for a, b, _ in evs)
    dec_ms = sorted(a.elapsed_time(c) for a, _, c in evs)
    kmean = sum(tile_ms) / len(tile_ms)          # the tile kernel (dominant)
    dmean = sum(dec_ms) / len(dec_ms)            # tile + merge kernels
    pct = lambda xs, p: xs[min(len(xs) - 1, int(round(p * (len(xs) - 1))))]
    log(f"step {ms_per_step * 1e3:.1f} us wall, decode {dmean * 1e3:.1f} us "
        f"(p10 {pct(dec_ms, 0.1) * 1e3:.1f}, p50 {pct(dec_ms, 0.5) * 1e3:.1f}, "
        f"p90 {pct(dec_ms, 0.9) * 1e3:.1f}), tile kernel {kmean * 1e3:.1f} us")

    # NEXT: device-planned step (no host plan, no upload), eager and as a
    # replayed HIP graph (its arguments are fixed; lengths live on the device)
    pa = dev.params_auto(tl, W)

    def step_auto(s):
        kp, vp = copies[s % len(copies)]
        # the current stream: the launch stream, or the capture stream inside torch.cuda.graph
        hda.hda_decode_auto(pa, dev.t["q"], kp, vp, dev.t["block_table"], dev.t["seq_lens"],
                            tl, W, out, torch.cuda.current_stream())

    for s in range(args.warmup):
        step_auto(s)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step_auto(s)
    torch.cuda.synchronize()
    auto_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    graphs = []
    for c in range(len(copies)):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            step_auto(c)
        graphs.append(gr)
    graphs[0].replay()                 # the replayed step reproduces the eager output
    torch.cuda.synchronize()
    o_graph = out.clone()
    step_auto(0)
    torch.cuda.synchronize()
    if not torch.equal(o_graph, out):
        raise RuntimeError("graph replay differs from the eager device-planned step")
    for s in range(args.warmup):
        graphs[s % len(graphs)].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        graphs[s % len(graphs)].replay()
    torch.cuda.synchronize()
    graph_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    # several steps per graph: each graph launch costs a gap of its own
    # before the next one starts (kernel trace: ~9 us), which a graph of
    # many launches -- a model step's layers -- pays once
    per_graph = 8
    gmany = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gmany):
        for s in range(per_graph):
            step_auto(s)
    gmany.replay()
    torch.cuda.synchronize()
    if not torch.equal(o_graph, out):      # every KV copy holds the same values
        raise RuntimeError("multi-step graph replay differs from the eager step")
    n_rep = max(1, args.steps // per_graph)
    t0 = time.perf_counter()
    for _ in range(n_rep):
        gmany.replay()
    torch.cuda.synchronize()
    graph8_ms = (time.perf_counter() - t0) * 1e3 / (n_rep * per_graph)
    log(f"device-planned step {auto_ms * 1e3:.1f} us wall, as HIP graph {graph_ms * 1e3:.1f} us "
        f"(one step per graph), {graph8_ms * 1e3:.1f} us ({per_graph} steps per graph)")
    del graphs, gmany

    # consistency check of the timed output (HIP path only; parity against
    # the oracle is the tests' job): a static 4-way split of the same batch
    # must reach the same attention
    o_static = dev.decode(hda.hda_plan_static(lens, 4))
    torch.cuda.synchronize()
    static_diff = float((o_static - out).abs().max())
    log(f"dynamic vs static-4 plan: max |diff| {static_diff:.3e}")
    del o_static

    algo = algorithmic_bytes(inp, plan_len)
    achieved = algo / (kmean * 1e-3) / 1e9
    traffic = traffic_from_profiles(args.workload)
    res = {
        # the headline metric names its mix; other decode mixes say theirs
        "metric": METRIC if args.workload == "extreme" else
                  f"decode-attn µs/step + KV GB/s (% HBM peak), {args.workload} mix, 1 GPU",
        "value": round(kv / (ms_per_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.kv_dtype == "bf16" else "fp8",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: " + (
            "1x131072 + 31x4096 KV tokens" if args.workload == "extreme" else
            f"{len(lens)} requests, {int(lens.sum())} KV tokens"),
            "batch": int(len(lens)), "kv_tokens": int(lens.sum()),
            "q_heads": w.n_q_heads, "kv_heads": w.n_kv_heads, "head_dim": w.head_dim,
            "page_size": w.page_size, "kv_dtype": w.kv_dtype, "kv_scale": inp["scale_mode"],
            "math": args.math,
            "tile_len": tl,
            "n_workgroups": W, "kv_bytes": kv},
        "us_per_step": {"wall": round(ms_per_step * 1e3, 2),
                        "decode_mean": round(dmean * 1e3, 2),
                        "decode_p10": round(pct(dec_ms, 0.1) * 1e3, 2),
                        "decode_p50": round(pct(dec_ms, 0.5) * 1e3, 2),
                        "decode_p90": round(pct(dec_ms, 0.9) * 1e3, 2),
                        "tile_kernel_mean": round(kmean * 1e3, 2),
                        "merge_and_gap_mean": round((dmean - kmean) * 1e3, 2)},
        "kv_gbs_decode": round(kv / (dmean * 1e-3) / 1e9, 2),
        "hbm_peak_frac_decode": round(kv / (dmean * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes": algo,
                     "kernel": ("hda_decode_argplan_kernel (tile kernel, plan in its launch "
                                "arguments; HIP events on its stream)" if upload_mode == "args" else
                                "hda_decode_kernel (tile kernel; HIP events on its stream)")},
        "plan": {"host_us": round(host_plan_us, 2), "upload_us": round(upload_us, 2),
                 "upload": upload_mode,
                 "plan_ints": int(n_plan)},
        "max_abs_diff_vs_static4_plan": static_diff,
        "device_planned_step": {"wall_us": round(auto_ms * 1e3, 2),
                                "graph_replay_wall_us": round(graph_ms * 1e3, 2),
                                "graph_8_steps_per_graph_wall_us": round(graph8_ms * 1e3, 2),
                                "kv_gbs_graph_8": round(kv / (graph8_ms * 1e-3) / 1e9, 2)},
    }

    if not args.no_read_probe:
        res["read_probe"] = read_probe(algo)
        log(f"read probe: {res['read_probe']['gbs']:.0f} GB/s reading the same "
            f"{algo / 1e9:.2f} GB ({res['read_probe']['n_workgroups']} workgroups); the tile "
            f"kernel reaches {achieved / res['read_probe']['gbs']:.1%} of it")

    if args.copy_probe:
        # a plain copy kernel of known size: reads and writes 2^30 bytes per
        # launch; the HBM counters of this launch calibrate the kernel's
        nbytes = 1 << 30
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        dst.copy_(src)
        e0.record()
        for _ in range(5):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 5
        res["copy_probe"] = {"bytes_read": nbytes, "bytes_written": nbytes,
                             "us": round(ms * 1e3, 2),
                             "read_plus_write_gbs": round(2 * nbytes / (ms * 1e-3) / 1e9, 1)}
        log(f"copy probe: 1 GiB copy {ms * 1e3:.1f} us")
        del src, dst

    if not args.no_static:
        # every plan timed the same way (events around the whole hda_decode
        # call, plan in device memory), the dynamic one included
        dyn = time_plan_kernel(dev, hda.hda_plan(lens, tl, W), copies, steps=8, warmup=2)
        dyn_ms = sum(dyn) / len(dyn)
        log(f"dynamic (tile_len {tl}, W {W}): {dyn_ms * 1e3:.1f} us")
        static = {}
        for S in (1, 2, 4, 8, 16, 32, 64):
            plan = hda.hda_plan_static(lens, S)
            ms = time_plan_kernel(dev, plan, copies, steps=8, warmup=2)
            static[S] = sum(ms) / len(ms)
            log(f"static S={S}: {static[S] * 1e3:.1f} us")
        best = min(static, key=static.get)
        S_h = max(1, min(64, math.ceil(256 * 2 / (len(lens) * w.n_kv_heads))))
        S_h = 1 << (S_h - 1).bit_length()
        # a static split is as slow as its longest chunk: one workgroup
        # streaming max(len)/S tokens of one kv head (K and V)
        one_wg = single_stream_gbs()
        per_tok = 2 * w.head_dim * (1 if w.kv_dtype == "fp8" else 2)
        predicted = {S: math.ceil(int(lens.max()) / S) * per_tok / (one_wg * 1e9) * 1e6
                     for S in static}
        log(f"one workgroup streams {one_wg:.1f} GB/s alone; static S=1 predicted "
            f"{predicted[1]:.0f} us from its longest chunk")
        res["load_balance"] = {
            "single_workgroup_gbs": round(one_wg, 2),
            "static_predicted_us": {str(k): round(v, 1) for k, v in predicted.items()},
            "dynamic_decode_us": round(dyn_ms * 1e3, 2),
            "static_us": {str(k): round(v * 1e3, 2) for k, v in static.items()},
            "static_best_S": best,
            "gain_vs_best_static": round(static[best] / dyn_ms, 3),
            "static_heuristic_S": S_h,
            "gain_vs_heuristic_static": round(static[S_h] / dyn_ms, 3),
            "timing": "events around each whole hda_decode call, plan in device memory, "
                      "KV copies rotated; the same for every plan",
        }

    if not args.no_cpu:
        log("timing the fp64 oracle on a bounded sample")
        res["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
        if args.workload == "extreme":
            # the oracle on one thread, on the two smallest workloads
            one = {}
            for name, budget in (("tiny", 2.0), ("uniform", 4.0)):
                small = make_inputs(CONFIGS[name])
                one[name] = cpu_baseline(small, budget, one_thread=True)
                log(f"oracle, 1 thread, {name}: {one[name]['value']} GB/s")
            res["cpu_baseline"]["one_thread"] = one

    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

"""Oracle decode attention over a paged KV cache (test infrastructure).

The method speeds up an exact computation: splitting a request's KV range
into tiles and combining the per-tile partial results reaches the same
softmax attention as processing the range in one piece ([ES-why]: the KV work
is cut into tiles; [EN-vllm]: it replaces a fixed split-KV schedule).  So the
oracle is the plain definition, in float64, from the exact stored values:

    out[b, h, :] = sum_{t < len_b} softmax_t(sm_scale * q[b, h] . K_b[t, kv(h)]) V_b[t, kv(h), :]

Readings taken where the pages are silent:
  * one query token per request; no mask inside [0, len_b) (the query sees
    every cached token, including the new one once it is written);
  * grouped-query heads: q head h reads kv head kv(h) = floor(h * Hkv / Hq)
    (consecutive q heads share a kv head);
  * cache layout: pages [n_pages][Hkv][page_size][D], separate K and V pools;
    token t of request b is row t mod page_size of page
    block_table[b][floor(t / page_size)];
  * per-tile partials are (o = normalised output, lse = natural-log
    log-sum-exp of the scaled scores) and are merged by log-sum-exp weights
    in slot order;
  * dequantisation scales: the pages name quantisation scales as a
    model-specific parameter ([ES-lim]) without fixing their granularity.
    A stored element's value is decode(code) * scale * extra, where scale is
    the per-tensor scalar (k_scale / v_scale) and extra is 1 ("tensor"),
    the element's kv head entry of a [Hkv] array ("head"), or the
    [n_pages, Hkv] array entry of the physical page and kv head holding the
    row ("page").
"""

import math
import numpy as np

from .codec import bf16_to_f64, fp8_decode


def decode_kv(raw, kv_dtype, scale=1.0):
    """Stored cache values -> float64: the decoded element times its scale
    (a scalar, or an array that broadcasts against raw)."""
    if kv_dtype == "bf16":
        return bf16_to_f64(raw) * np.asarray(scale, dtype=np.float64)
    if kv_dtype == "fp8":
        return fp8_decode(raw) * np.asarray(scale, dtype=np.float64)
    raise ValueError(kv_dtype)


SCALE_MODES = ("tensor", "head", "page")


def row_scales(scale, scale_mode, scales, block_table_row, length, page_size, n_kv_heads):
    """Dequantisation scale of each cached row of one request, per kv head:
    float64 [length, Hkv] (see the module docstring for the three modes)."""
    base = np.full((length, n_kv_heads), np.float64(scale))
    if scale_mode == "tensor":
        return base
    if scale_mode == "head":
        return base * np.asarray(scales, dtype=np.float64)[None, :]
    if scale_mode == "page":
        t = np.arange(length)
        pages = np.asarray(block_table_row, dtype=np.int64)[t // page_size]
        return base * np.asarray(scales, dtype=np.float64)[pages]
    raise ValueError(scale_mode)


def gather_request(pages, block_table_row, length, page_size):
    """Raw rows of one request in token order: [length, Hkv, D]."""
    n_pages = (length + page_size - 1) // page_size
    ids = np.asarray(block_table_row[:n_pages], dtype=np.int64)
    g = pages[ids]                               # [n_pages, Hkv, ps, D]
    g = np.transpose(g, (0, 2, 1, 3))            # [n_pages, ps, Hkv, D]
    g = g.reshape(n_pages * page_size, g.shape[2], g.shape[3])
    return g[:length]


def _kv_head(h, n_q_heads, n_kv_heads):
    return (h * n_kv_heads) // n_q_heads


def _attend_one(q_rows, k, v, sm_scale):
    """Softmax attention of q_rows [g, D] over k, v [L, D], all float64."""
    s = (k @ q_rows.T) * sm_scale                # [L, g]
    s = s - s.max(axis=0, keepdims=True)
    w = np.exp(s)
    return (w.T @ v) / w.sum(axis=0)[:, None]    # [g, D]


def attention_reference(q, k_pages, v_pages, block_table, seq_lens, kv_dtype,
                        sm_scale, k_scale=1.0, v_scale=1.0, scale_mode="tensor",
                        k_scales=None, v_scales=None):
    """Exact attention for every request and q head.  q: float64 [B, Hq, D].

    Requests are processed one kv head at a time so that host memory stays
    bounded by one request's K and V slice in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv, ps = k_pages.shape[1], k_pages.shape[2]
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        kr = gather_request(k_pages, block_table[b], L, ps)
        vr = gather_request(v_pages, block_table[b], L, ps)
        ks = row_scales(k_scale, scale_mode, k_scales, block_table[b], L, ps, Hkv)
        vs = row_scales(v_scale, scale_mode, v_scales, block_table[b], L, ps, Hkv)
        for kvh in range(Hkv):
            heads = [h for h in range(Hq) if _kv_head(h, Hq, Hkv) == kvh]
            k = decode_kv(kr[:, kvh, :], kv_dtype, ks[:, kvh, None])
            v = decode_kv(vr[:, kvh, :], kv_dtype, vs[:, kvh, None])
            out[b, heads] = _attend_one(q[b, heads], k, v, sm_scale)
    return out


def attention_selected(q, k_pages, v_pages, block_table, seq_lens, kv_dtype,
                       sm_scale, pairs, k_scale=1.0, v_scale=1.0, scale_mode="tensor",
                       k_scales=None, v_scales=None):
    """The same definition for selected (b, h) pairs only -> {(b, h): [D]}."""
    q = np.asarray(q, dtype=np.float64)
    Hq = q.shape[1]
    Hkv, ps = k_pages.shape[1], k_pages.shape[2]
    res = {}
    for (b, h) in pairs:
        L = int(seq_lens[b])
        kvh = _kv_head(h, Hq, Hkv)
        ks = row_scales(k_scale, scale_mode, k_scales, block_table[b], L, ps, Hkv)
        vs = row_scales(v_scale, scale_mode, v_scales, block_table[b], L, ps, Hkv)
        k = decode_kv(gather_request(k_pages, block_table[b], L, ps)[:, kvh, :], kv_dtype,
                      ks[:, kvh, None])
        v = decode_kv(gather_request(v_pages, block_table[b], L, ps)[:, kvh, :], kv_dtype,
                      vs[:, kvh, None])
        res[(b, h)] = _attend_one(q[b, [h]], k, v, sm_scale)[0]
    return res


def attention_bruteforce(q, k_pages, v_pages, block_table, seq_lens, kv_dtype,
                         sm_scale, k_scale=1.0, v_scale=1.0, scale_mode="tensor",
                         k_scales=None, v_scales=None):
    """Pure-Python triple loop with math.fsum; for tiny inputs only.

    Reads each token through its own page lookup (no gather) and looks up
    its scale from the page id and kv head itself, so that it shares neither
    the gather/reshape path nor the row-scale helper of attention_reference.
    """
    qf = np.asarray(q, dtype=np.float64).tolist()
    B, Hq, D = len(qf), len(qf[0]), len(qf[0][0])
    Hkv, ps = k_pages.shape[1], k_pages.shape[2]
    kd = decode_kv(k_pages, kv_dtype).tolist()
    vd = decode_kv(v_pages, kv_dtype).tolist()
    bt = np.asarray(block_table).tolist()
    ksl = None if k_scales is None else np.asarray(k_scales, dtype=np.float64).tolist()
    vsl = None if v_scales is None else np.asarray(v_scales, dtype=np.float64).tolist()

    def scale_of(base, arr, page, kvh):
        if scale_mode == "tensor":
            return float(base)
        if scale_mode == "head":
            return float(base) * arr[kvh]
        if scale_mode == "page":
            return float(base) * arr[page][kvh]
        raise ValueError(scale_mode)

    out = [[[0.0] * D for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        L = int(seq_lens[b])
        for h in range(Hq):
            kvh = (h * Hkv) // Hq
            scores = []
            for t in range(L):
                page, row = bt[b][t // ps], t % ps
                krow = kd[page][kvh][row]
                ks = scale_of(k_scale, ksl, page, kvh)
                scores.append(sm_scale * math.fsum(qf[b][h][d] * krow[d] * ks for d in range(D)))
            m = max(scores)
            w = [math.exp(s - m) for s in scores]
            z = math.fsum(w)
            for d in range(D):
                acc = math.fsum(w[t] * vd[bt[b][t // ps]][kvh][t % ps][d]
                                * scale_of(v_scale, vsl, bt[b][t // ps], kvh) for t in range(L))
                out[b][h][d] = acc / z
    return np.array(out, dtype=np.float64)


def split_merge_reference(q, k_pages, v_pages, block_table, seq_lens, kv_dtype,
                          sm_scale, plan, k_scale=1.0, v_scale=1.0, scale_mode="tensor",
                          k_scales=None, v_scales=None):
    """Attention computed the way a plan splits it, in float64.

    For each item (b, kv_begin, kv_end, slot) and q head: m = max score,
    l = sum exp(s - m), o = sum exp(s - m) v / l, lse = m + ln l.  Items with
    slot -1 give the output directly; otherwise the request's partials are
    combined in slot order with weights exp(lse_p - max_p lse_p).
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv, ps = k_pages.shape[1], k_pages.shape[2]
    out = np.full((B, Hq, D), np.nan)
    P = plan.n_partials
    part_o = np.full((P, Hq, D), np.nan)
    part_lse = np.full((P, Hq), np.nan)
    cache = {}
    for (b, k0, k1, slot) in plan.items:
        if b not in cache:
            L = int(seq_lens[b])
            cache = {b: (gather_request(k_pages, block_table[b], L, ps),
                         gather_request(v_pages, block_table[b], L, ps),
                         row_scales(k_scale, scale_mode, k_scales, block_table[b], L, ps, Hkv),
                         row_scales(v_scale, scale_mode, v_scales, block_table[b], L, ps, Hkv))}
        kr, vr, ks, vs = cache[b]
        for h in range(Hq):
            kvh = _kv_head(h, Hq, Hkv)
            k = decode_kv(kr[k0:k1, kvh, :], kv_dtype, ks[k0:k1, kvh, None])
            v = decode_kv(vr[k0:k1, kvh, :], kv_dtype, vs[k0:k1, kvh, None])
            s = (k @ q[b, h]) * sm_scale
            m = s.max()
            e = np.exp(s - m)
            l = e.sum()
            o = (e @ v) / l
            if slot < 0:
                out[b, h] = o
            else:
                part_o[slot, h] = o
                part_lse[slot, h] = m + math.log(l)
    for b in range(B):
        s0, s1 = plan.req_part_ptr[b], plan.req_part_ptr[b + 1]
        if s1 == s0:
            continue
        for h in range(Hq):
            lse = part_lse[s0:s1, h]
            M = lse.max()
            wts = np.exp(lse - M)
            out[b, h] = (wts @ part_o[s0:s1, h]) / wts.sum()
    return out

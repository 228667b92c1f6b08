"""Oracle for multi-token (prefill / chunked-prefill) attention over the
paged cache (test infrastructure).

The backend's attention also serves the prefill phase: the pages report it
cutting time to first token ([ES-why]; the arex-research page's merge note;
[EN-vllm]'s summary) but give no prefill algorithm.  Readings taken:

  * request b brings q_len_b new query tokens whose K and V are already in
    the cache, which then holds kv_len_b >= q_len_b tokens; query row r sits
    at position pos = kv_len_b - q_len_b + r;
  * causal attention: row r attends to cache tokens 0..pos (itself
    included, as a decode query attends to its own new token), nothing
    after;
  * q is packed request after request: [sum_b q_len_b][Hq][D]; the output
    has the same layout.

prefill_reference is that definition in float64.  prefill_rows is the
row-block rule the planner is fed with: the query rows of a request are
grouped, in order, into blocks of rows_per_block rows (the last one
shorter); a block whose last row sits at position p needs cache tokens
[0, p + 1), which becomes the block's length for the same tile planner as
decode.
"""

import math

import numpy as np

from .attention import decode_kv, gather_request, row_scales, _kv_head


def q_offsets(q_lens):
    """Start row of each request's queries in the packed q: [B + 1]."""
    return np.concatenate([[0], np.cumsum(np.asarray(q_lens, dtype=np.int64))])


def prefill_reference(q, k_pages, v_pages, block_table, kv_lens, q_lens, kv_dtype, sm_scale,
                      k_scale=1.0, v_scale=1.0, scale_mode="tensor", k_scales=None,
                      v_scales=None):
    """Causal attention for every packed query row and q head, float64.
    q: float64 [sum q_len][Hq][D]."""
    q = np.asarray(q, dtype=np.float64)
    Hq = q.shape[1]
    Hkv, ps = k_pages.shape[1], k_pages.shape[2]
    off = q_offsets(q_lens)
    out = np.full(q.shape, np.nan)
    for b in range(len(q_lens)):
        L, n = int(kv_lens[b]), int(q_lens[b])
        kr = gather_request(k_pages, block_table[b], L, ps)
        vr = gather_request(v_pages, block_table[b], L, ps)
        ks = row_scales(k_scale, scale_mode, k_scales, block_table[b], L, ps, Hkv)
        vs = row_scales(v_scale, scale_mode, v_scales, block_table[b], L, ps, Hkv)
        for kvh in range(Hkv):
            k = decode_kv(kr[:, kvh, :], kv_dtype, ks[:, kvh, None])
            v = decode_kv(vr[:, kvh, :], kv_dtype, vs[:, kvh, None])
            heads = [h for h in range(Hq) if _kv_head(h, Hq, Hkv) == kvh]
            for r in range(n):
                pos = L - n + r
                qr = q[off[b] + r, heads]                       # [g, D]
                s = (k[:pos + 1] @ qr.T) * sm_scale             # [pos+1, g]
                s = s - s.max(axis=0, keepdims=True)
                w = np.exp(s)
                out[off[b] + r, heads] = (w.T @ v[:pos + 1]) / w.sum(axis=0)[:, None]
    return out


def prefill_rows(q_lens, kv_lens, rows_per_block):
    """Row blocks in order: list of (b, first packed row, rows, position of
    the first row), and each block's causal extent (its planner length)."""
    off = q_offsets(q_lens)
    rows, extents = [], []
    for b, (n, L) in enumerate(zip(np.asarray(q_lens).tolist(), np.asarray(kv_lens).tolist())):
        for q0 in range(0, n, rows_per_block):
            nq = min(rows_per_block, n - q0)
            pos0 = L - n + q0
            rows.append((b, int(off[b]) + q0, nq, pos0))
            extents.append(pos0 + nq)
    return rows, extents

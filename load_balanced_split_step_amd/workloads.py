"""Seeded synthetic decode workloads (input generation only).

This module draws inputs and nothing else: it holds none of the attention,
planning, normalisation or rotary arithmetic.  Both the HIP library's tests
and the fp64 oracle consume the byte arrays it returns.

Workloads, grouped-query attention over a paged cache (single-token decode
unless they bring several query rows):

  tiny      4 requests, lengths {17, 64, 200, 513}, 8 q / 2 kv heads, D 64,
            page 16, bf16, pages laid out contiguously
  uniform   32 requests x 4096 tokens, 64 q / 8 kv heads, D 128, page 64,
            bf16, pages randomly permuted in a shared pool
  extreme   one 131072-token request + 31 x 4096 (the 1 x 128K + 31 x 4K
            extreme mix the Dynamic Attention paragraphs of the arex-research
            page measure), otherwise as uniform
  longtail  64 requests, lengths log-uniform in [256, 65536], per-kv-head
            K and V scales drawn from U(0.5, 2), otherwise as uniform
  fp8       128 requests, lengths log-uniform in [1024, 32768], fp8 E4M3FN
            cache with per-tensor fp32 scales, and a new token per request
            that the fused prologue (RMSNorm with weights ~ N(1, 0.1),
            RoPE with theta 1e6) must write before attention reads it
  fp8_page  the long-tail lengths and per-head magnitudes, fp8 E4M3FN cache
            with one fp32 scale per (page, kv head) slab, and the prologue
  specdec   the extreme mix with 4 query rows per request (a speculative
            check of 3 draft tokens plus one), causal over the cache
  chunked   16 requests, cache lengths log-uniform in [2048, 32768], a
            chunk of U{16..128} new query rows each (chunked prefill)
  chunked_fp8  the same lengths and rows over an fp8 E4M3FN cache with
            per-tensor scales

Recipe (the pages use no dataset; these stand in for a serving batch):
  * numpy PCG64 streams spawned from SeedSequence(seed), one stream per
    quantity (lengths, page permutation, q, K, V, head scales, norm weights,
    new-token k/v); large tensors are drawn in fixed-size chunks, each from
    its own spawned child stream, so the bytes do not depend on threading;
  * values ~ N(0, 1) in float32, then rounded to bf16 by torch's
    round-to-nearest-even cast (a library conversion); optionally the V
    values of request b are multiplied by 2^-u_b, u_b ~ U(0, v_req_spread)
    (a stress case for scale granularity, drawn from its own stream);
  * log-uniform lengths: floor(exp(U(ln lo, ln hi))) clamped to [lo, hi];
  * random placement: the pool holds exactly sum_b ceil(len_b / page) pages
    and logical page p of request b lives in physical page
    perm[sum_{b'<b} pages_b' + p]; unused block-table entries are -1;
  * fp8: scale = amax / 448 in float32 over the drawn values of the whole
    pool ("tensor"), of one kv head ("head") or of one (page, kv head) slab
    ("page"); codes from torch's float8_e4m3fn cast of clip(x / scale, +-448);
    a bf16 cache with "head" scales stores bf16(x / scale) with the same
    per-head scales (no scale otherwise);
  * rows past len_b in a request's last page hold NaN (when poisoned), and
    for the prologue workload so does the new token's slot len_b - 1.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Optional, Sequence, Tuple

import numpy as np

BF16_NAN = np.uint16(0x7FC0)
FP8_NAN = np.uint8(0x7F)

# stream indices of SeedSequence(seed).spawn(...)
_S_LENS, _S_PERM, _S_Q, _S_K, _S_V, _S_HEADSCALE, _S_NORMW, _S_NEW, _S_SLABSCALE, _S_QLEN = range(10)
_N_STREAMS = 10


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    page_size: int
    kv_dtype: str = "bf16"              # "bf16" or "fp8"
    lengths: Optional[Tuple[int, ...]] = None
    len_range: Optional[Tuple[int, int]] = None   # log-uniform [lo, hi]
    placement: str = "random"           # "random" or "contiguous"
    head_scale: bool = False            # per-kv-head U(0.5, 2) on K and V
    prologue: bool = False              # new token written by the prologue
    kv_scale: str = "tensor"            # fp8 scale granularity: tensor, head, page
    v_req_spread: float = 0.0           # per-request V magnitude 2^-U(0, spread)
    # multi-token queries (prefill / chunked prefill): q_len per request, or
    # drawn uniformly from q_len_range; the cache lengths include them
    q_lens: Optional[Tuple[int, ...]] = None
    q_len_range: Optional[Tuple[int, int]] = None
    seed: int = 0
    rms_eps: float = 1e-6
    rope_theta: float = 1e6

    @property
    def group(self):
        return self.n_q_heads // self.n_kv_heads

    @property
    def prefill(self):
        return self.q_lens is not None or self.q_len_range is not None

    def with_(self, **kw):
        return replace(self, **kw)


CONFIGS = {
    "tiny": Workload("tiny", 4, 8, 2, 64, 16, lengths=(17, 64, 200, 513),
                     placement="contiguous", seed=0),
    "uniform": Workload("uniform", 32, 64, 8, 128, 64, lengths=(4096,) * 32, seed=1),
    "extreme": Workload("extreme", 32, 64, 8, 128, 64,
                        lengths=(131072,) + (4096,) * 31, seed=2),
    "longtail": Workload("longtail", 64, 64, 8, 128, 64, len_range=(256, 65536),
                         head_scale=True, seed=3),
    "fp8": Workload("fp8", 128, 64, 8, 128, 64, kv_dtype="fp8",
                    len_range=(1024, 32768), prologue=True, seed=4),
    "fp8_page": Workload("fp8_page", 64, 64, 8, 128, 64, kv_dtype="fp8",
                         len_range=(256, 65536), head_scale=True, prologue=True,
                         kv_scale="page", seed=5),
    # multi-token queries over the cache (lengths include the new rows)
    "specdec": Workload("specdec", 32, 64, 8, 128, 64, lengths=(131072,) + (4096,) * 31,
                        q_lens=(4,) * 32, seed=6),
    "chunked": Workload("chunked", 16, 64, 8, 128, 64, len_range=(2048, 32768),
                        q_len_range=(16, 128), seed=7),
    "chunked_fp8": Workload("chunked_fp8", 16, 64, 8, 128, 64, kv_dtype="fp8",
                            len_range=(2048, 32768), q_len_range=(16, 128), seed=7),
}

_CHUNK_SLABS = 256


def _threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _bf16_bits(x):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _fp8_bits(x):
    import torch
    x = np.clip(np.asarray(x, dtype=np.float32), -448.0, 448.0)
    return torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _rng(ss):
    return np.random.Generator(np.random.PCG64(ss))


def draw_lengths(w: Workload, seed: int):
    if w.lengths is not None:
        lens = np.array(w.lengths, dtype=np.int64)
        assert len(lens) == w.batch
        return lens.astype(np.int32)
    lo, hi = w.len_range
    r = _rng(np.random.SeedSequence(seed).spawn(_N_STREAMS)[_S_LENS])
    u = r.uniform(math.log(lo), math.log(hi), size=w.batch)
    return np.clip(np.floor(np.exp(u)), lo, hi).astype(np.int32)


def _draw_pool(ss, n_pages, w: Workload, head_scales, fp8_scale=None, slab_mult=None):
    """One page pool [n_pages, Hkv, ps, D], drawn in chunks of whole
    (page, head) slabs.

    For an fp8 cache with "tensor" or "head" scales this runs twice: first
    with fp8_scale None, returning the float32 amax per kv head [Hkv]; then
    with the scale (a scalar, or [Hkv]), returning the stored bits.  With
    "page" scales one pass returns (bits, scales [n_pages, Hkv]), each slab's
    scale being its own amax / 448.  A bf16 cache returns the bits."""
    Hkv, ps, D = w.n_kv_heads, w.page_size, w.head_dim
    slab = ps * D
    n_slabs = n_pages * Hkv
    n_chunks = max(1, (n_slabs + _CHUNK_SLABS - 1) // _CHUNK_SLABS)
    # child c of ss, built from its spawn key: the same streams on every pass
    # (ss.spawn would hand out new children on a second call)
    children = [np.random.SeedSequence(ss.entropy, spawn_key=ss.spawn_key + (c,))
                for c in range(n_chunks)]
    fp8 = w.kv_dtype == "fp8"
    scaled = fp8 or w.kv_scale != "tensor"     # a bf16 cache may carry head scales
    page_mode = fp8 and w.kv_scale == "page"
    amax_pass = scaled and not page_mode and fp8_scale is None
    if not amax_pass:
        out = np.empty((n_slabs, slab), dtype=np.uint8 if fp8 else np.uint16)
    slab_scale = np.empty(n_slabs, dtype=np.float32) if page_mode else None
    if scaled and not page_mode and not amax_pass:
        fp8_scale = np.broadcast_to(np.asarray(fp8_scale, dtype=np.float32), (Hkv,))

    def work(c):
        s0 = c * _CHUNK_SLABS
        s1 = min(n_slabs, s0 + _CHUNK_SLABS)
        x = np.empty((s1 - s0, slab), dtype=np.float32)
        _rng(children[c]).standard_normal(out=x, dtype=np.float32)
        heads = np.arange(s0, s1) % Hkv
        if head_scales is not None:
            x *= head_scales[heads][:, None]
        if slab_mult is not None:
            x *= slab_mult[s0:s1][:, None]
        if amax_pass:
            am = np.abs(x).max(axis=1)
            return np.array([am[heads == h].max(initial=0.0) for h in range(Hkv)],
                            dtype=np.float32)
        if page_mode:
            sc = np.abs(x).max(axis=1) / np.float32(448.0)
            slab_scale[s0:s1] = sc
            out[s0:s1] = _fp8_bits(x / sc[:, None])
        elif fp8:
            out[s0:s1] = _fp8_bits(x / fp8_scale[heads][:, None])
        elif scaled:
            out[s0:s1] = _bf16_bits(x / fp8_scale[heads][:, None])
        else:
            out[s0:s1] = _bf16_bits(x)
        return None

    with ThreadPoolExecutor(_threads()) as ex:
        res = list(ex.map(work, range(n_chunks)))
    if amax_pass:
        return np.max(np.stack(res), axis=0).astype(np.float32)
    bits = out.reshape(n_pages, Hkv, ps, D)
    if page_mode:
        return bits, slab_scale.reshape(n_pages, Hkv)
    return bits


def draw_q_lens(w: Workload, seed: int, kv_lens):
    """Query rows per request for a multi-token workload (<= the cache length)."""
    if w.q_lens is not None:
        q = np.array(w.q_lens, dtype=np.int64)
        assert len(q) == len(kv_lens)
    else:
        lo, hi = w.q_len_range
        r = _rng(np.random.SeedSequence(seed).spawn(_N_STREAMS)[_S_QLEN])
        q = r.integers(lo, hi + 1, size=len(kv_lens))
    return np.minimum(q, np.asarray(kv_lens, dtype=np.int64)).astype(np.int32)


def make_inputs(w: Workload, seed: Optional[int] = None, poison: bool = True,
                lengths: Optional[Sequence[int]] = None,
                q_lens: Optional[Sequence[int]] = None):
    """Draw one decode batch.  Returns a dict of numpy arrays and scalars:

    q [B, Hq, D] u16 (bf16), k_pages / v_pages [NP, Hkv, ps, D] (u16 bf16 or
    u8 fp8), block_table [B, max_pages] i32, seq_lens [B] i32 (cache lengths),
    for a multi-token workload q_lens [B] i32 and q packed [sum q_lens, Hq, D], sm_scale,
    k_scale, v_scale (float32), scale_mode with k_scales / v_scales (None,
    float32 [Hkv] or [NP, Hkv]), and for the prologue workload q_norm_w,
    k_norm_w [D] u16, k_new, v_new [B, Hkv, D] u16, rms_eps, rope_theta.
    """
    seed = w.seed if seed is None else seed
    ss = np.random.SeedSequence(seed).spawn(_N_STREAMS)
    lens = (np.asarray(lengths, dtype=np.int32) if lengths is not None
            else draw_lengths(w, seed))
    B = len(lens)
    Hq, Hkv, D, ps = w.n_q_heads, w.n_kv_heads, w.head_dim, w.page_size
    assert Hq % Hkv == 0

    pages_per = (lens.astype(np.int64) + ps - 1) // ps
    n_pages = int(pages_per.sum())
    max_pages = int(pages_per.max())
    if w.placement == "contiguous":
        perm = np.arange(n_pages, dtype=np.int64)
    else:
        perm = _rng(ss[_S_PERM]).permutation(n_pages)
    block_table = np.full((B, max_pages), -1, dtype=np.int32)
    first = np.concatenate([[0], np.cumsum(pages_per)[:-1]])
    for b in range(B):
        block_table[b, :pages_per[b]] = perm[first[b]:first[b] + pages_per[b]]

    head_k = head_v = None
    if w.head_scale:
        hs = _rng(ss[_S_HEADSCALE]).uniform(0.5, 2.0, size=(2, Hkv)).astype(np.float32)
        head_k, head_v = hs[0], hs[1]

    mult_k = mult_v = None
    if w.v_req_spread > 0:
        # every page belongs to one request: its V slabs take that request's factor
        u = _rng(ss[_S_SLABSCALE]).uniform(0.0, w.v_req_spread, size=B)
        owner = np.empty(n_pages, dtype=np.int64)
        for b in range(B):
            owner[block_table[b, :pages_per[b]]] = b
        mult_v = np.repeat(np.exp2(-u).astype(np.float32)[owner], Hkv)
    k_scale = v_scale = np.float32(1.0)
    k_scales = v_scales = None
    scale_mode = w.kv_scale
    assert scale_mode in ("tensor", "head", "page")
    if w.kv_dtype == "bf16" and scale_mode == "page":
        raise ValueError("per-page scales are for an fp8 cache")
    k_ss, v_ss = ss[_S_K], ss[_S_V]
    if scale_mode == "page":
        k_pages, k_scales = _draw_pool(k_ss, n_pages, w, head_k, slab_mult=mult_k)
        v_pages, v_scales = _draw_pool(v_ss, n_pages, w, head_v, slab_mult=mult_v)
    else:
        if w.kv_dtype == "fp8" or scale_mode == "head":
            ka = _draw_pool(k_ss, n_pages, w, head_k, slab_mult=mult_k) / np.float32(448.0)
            va = _draw_pool(v_ss, n_pages, w, head_v, slab_mult=mult_v) / np.float32(448.0)
            if scale_mode == "head":
                k_scales, v_scales = ka.astype(np.float32), va.astype(np.float32)
            else:
                k_scale, v_scale = np.float32(ka.max()), np.float32(va.max())
        k_pages = _draw_pool(k_ss, n_pages, w, head_k,
                             fp8_scale=k_scales if scale_mode == "head" else k_scale,
                             slab_mult=mult_k)
        v_pages = _draw_pool(v_ss, n_pages, w, head_v,
                             fp8_scale=v_scales if scale_mode == "head" else v_scale,
                             slab_mult=mult_v)

    qlens = None
    if w.prefill or q_lens is not None:
        qlens = (np.minimum(np.asarray(q_lens, dtype=np.int32), lens) if q_lens is not None
                 else draw_q_lens(w, seed, lens))
        n_q = int(qlens.sum())
    else:
        n_q = B
    q = _bf16_bits(_rng(ss[_S_Q]).standard_normal((n_q, Hq, D), dtype=np.float32))

    inp = dict(workload=w, seed=seed, q=q, k_pages=k_pages, v_pages=v_pages,
               block_table=block_table, seq_lens=lens.astype(np.int32),
               sm_scale=np.float32(1.0 / math.sqrt(D)),
               k_scale=k_scale, v_scale=v_scale, kv_dtype=w.kv_dtype,
               scale_mode=scale_mode, k_scales=k_scales, v_scales=v_scales)
    if qlens is not None:
        inp["q_lens"] = qlens

    if w.prologue:
        r = _rng(ss[_S_NORMW])
        inp["q_norm_w"] = _bf16_bits(r.normal(1.0, 0.1, size=D).astype(np.float32))
        inp["k_norm_w"] = _bf16_bits(r.normal(1.0, 0.1, size=D).astype(np.float32))
        r = _rng(ss[_S_NEW])
        inp["k_new"] = _bf16_bits(r.standard_normal((B, Hkv, D), dtype=np.float32))
        inp["v_new"] = _bf16_bits(r.standard_normal((B, Hkv, D), dtype=np.float32))
        inp["rms_eps"] = np.float32(w.rms_eps)
        inp["rope_theta"] = np.float32(w.rope_theta)

    if poison:
        nan = FP8_NAN if w.kv_dtype == "fp8" else BF16_NAN
        for b in range(B):
            L = int(lens[b])
            first_bad = L - 1 if w.prologue else L
            last_page = (L - 1) // ps
            for t in range(first_bad, (last_page + 1) * ps):
                pg = block_table[b, t // ps]
                k_pages[pg, :, t % ps, :] = nan
                v_pages[pg, :, t % ps, :] = nan
    return inp


def kv_bytes(inp):
    """Algorithmic KV bytes one decode step must read: every cached token's
    K and V row for every kv head."""
    w = inp["workload"]
    elem = 1 if w.kv_dtype == "fp8" else 2
    return int(np.asarray(inp["seq_lens"], dtype=np.int64).sum()) * w.n_kv_heads * w.head_dim * 2 * elem


# ---- Router GEMM inputs ----

@dataclass(frozen=True)
class RouterWorkload:
    """Router logits x w^T: bf16 activations [tokens][hidden], fp32 weights
    [experts][hidden] ~ N(0, 1/hidden) so that logits are ~ N(0, 1)."""
    name: str
    tokens: int
    hidden: int
    experts: int
    seed: int = 0

    def with_(self, **kw):
        return replace(self, **kw)


ROUTER_CONFIGS = {
    "router_small": RouterWorkload("router_small", 5, 96, 24, seed=20),
    # DeepSeek-V3-like router shape (hidden 7168, 256 experts); the pages do
    # not give Hy3's router shape; token counts span decode to prefill
    "router": RouterWorkload("router", 64, 7168, 256, seed=21),
}


def make_router_inputs(w: RouterWorkload, tokens: Optional[int] = None):
    """x bf16 bits [T][H] ~ N(0, 1), weights fp32 [E][H] ~ N(0, 1/H)."""
    T = w.tokens if tokens is None else tokens
    ss = np.random.SeedSequence(w.seed).spawn(2)
    x = _bf16_bits(_rng(ss[0]).standard_normal((T, w.hidden), dtype=np.float32))
    wt = (_rng(ss[1]).standard_normal((w.experts, w.hidden), dtype=np.float32)
          * np.float32(1.0 / math.sqrt(w.hidden))).astype(np.float32)
    return dict(workload=w, x=x, w=wt)

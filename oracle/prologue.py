"""Oracle for the new-token prologue: QK-RMSNorm, RoPE, KV write
(test infrastructure).

The attention backend puts a fused "RoPE + QK-Norm + KV-write" prologue in
front of the attention ([EN-vllm]); the pages give none of its details and
list rotary embeddings, normalisation order, head dims, quantisation scales
and cache layouts as model-specific integration work ([ES-lim]).

Readings taken:
  * order: RMSNorm first, then RoPE (norm with per-dimension weights and a
    rotation do not commute, so the order matters);
  * RMSNorm per head over D: y = x / sqrt(mean_d(x^2) + eps) * w, one weight
    vector [D] for q and another for k, shared by all heads;
  * RoPE in the rotate-half form over the full head dim: for i < D/2,
    phi_i = pos * theta^(-2i/D), and the pair (x_i, x_{i+D/2}) is rotated by
    phi_i.  The interleaved-pair form is provided for tests that tell the
    two apart;
  * the new token sits at position pos = len_b - 1 (len_b counts it); its k
    (normalised and rotated) and v are stored into that cache slot, in the
    cache format as x / scale: fp8 codes, or bf16 rounded to nearest-even.
    The scale is the one the attention reads that slot with: the per-tensor
    scalar times, per the scale mode, the kv head's entry ("head") or the
    (physical page of the slot, kv head) entry ("page") -- an existing
    page's scale is not changed by the write;
  * attention then uses the normalised, rotated q.
"""

import numpy as np

from .codec import bf16_to_f64, fp8_encode


def rms_norm(x, w, eps):
    """RMSNorm over the last axis, float64."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(w, dtype=np.float64)


def rope(x, pos, theta, style="rotate_half"):
    """Rotary embedding of x [..., D] at position(s) pos (broadcast over the
    leading axes), float64."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    half = D // 2
    i = np.arange(half, dtype=np.float64)
    inv_freq = theta ** (-2.0 * i / D)
    pos = np.asarray(pos, dtype=np.float64)
    phi = pos[..., None] * inv_freq                  # [..., D/2]
    c, s = np.cos(phi), np.sin(phi)
    y = np.empty_like(x)
    if style == "rotate_half":
        a, b = x[..., :half], x[..., half:]
        y[..., :half] = a * c - b * s
        y[..., half:] = b * c + a * s
    elif style == "interleaved":
        a, b = x[..., 0::2], x[..., 1::2]
        y[..., 0::2] = a * c - b * s
        y[..., 1::2] = b * c + a * s
    else:
        raise ValueError(style)
    return y


def bf16_encode(x):
    """float64 -> bf16 bit patterns, round to nearest, ties to even.

    Rounds the significand directly from float64 (no detour through float32,
    which could round twice).  Only the normal bf16 range is needed here.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                         # x = m * 2^e, 0.5 <= |m| < 1
    q = np.rint(m * 256.0)                     # 8 significant bits, half-to-even
    v = np.ldexp(q, e - 8)
    nz = v != 0
    assert np.all(np.abs(v[nz]) >= 2.0 ** -126) and np.all(np.abs(v) < 3.0e38), \
        "bf16_encode: value outside the normal bf16 range"
    return (v.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def slot_scales(scale, scale_mode, scales, block_table, seq_lens, page_size, n_kv_heads):
    """Scale of the new token's cache slot (row len_b - 1) per request and
    kv head: float64 [B, Hkv]."""
    B = len(seq_lens)
    out = np.full((B, n_kv_heads), np.float64(scale))
    if scale_mode == "tensor":
        return out
    arr = np.asarray(scales, dtype=np.float64)
    if scale_mode == "head":
        return out * arr[None, :]
    if scale_mode == "page":
        for b, L in enumerate(np.asarray(seq_lens).tolist()):
            page = int(block_table[b][(L - 1) // page_size])
            out[b] *= arr[page]
        return out
    raise ValueError(scale_mode)


def prologue_step(q, k_new, v_new, q_norm_w, k_norm_w, seq_lens, rms_eps,
                  rope_theta, kv_dtype, k_scale=1.0, v_scale=1.0, scale_mode="tensor",
                  k_scales=None, v_scales=None, block_table=None, page_size=None):
    """Returns (q', k', v, k_codes, v_codes) for the new token of each request.

    q: bf16 bits [B, Hq, D]; k_new, v_new: bf16 bits [B, Hkv, D];
    q_norm_w, k_norm_w: bf16 bits [D].  With "head" or "page" scales,
    k_scales / v_scales hold the per-head or per-(page, head) factors, and
    the "page" mode also needs block_table and page_size to find the slot.
    """
    pos = np.asarray(seq_lens, dtype=np.int64) - 1
    qf = bf16_to_f64(q)
    kf = bf16_to_f64(k_new)
    vf = bf16_to_f64(v_new)
    wq = bf16_to_f64(q_norm_w)
    wk = bf16_to_f64(k_norm_w)
    q_p = rope(rms_norm(qf, wq, rms_eps), pos[:, None], rope_theta)
    k_p = rope(rms_norm(kf, wk, rms_eps), pos[:, None], rope_theta)
    Hkv = kf.shape[1]
    ks = slot_scales(k_scale, scale_mode, k_scales, block_table, seq_lens, page_size, Hkv)
    vs = slot_scales(v_scale, scale_mode, v_scales, block_table, seq_lens, page_size, Hkv)
    if kv_dtype == "fp8":
        k_codes = fp8_encode(k_p / ks[:, :, None])
        v_codes = fp8_encode(vf / vs[:, :, None])
    elif kv_dtype == "bf16":
        k_codes = bf16_encode(k_p / ks[:, :, None])
        v_codes = bf16_encode(vf / vs[:, :, None])
    else:
        raise ValueError(kv_dtype)
    return q_p, k_p, vf, k_codes, v_codes


def write_new_token(k_pages, v_pages, block_table, seq_lens, k_codes, v_codes):
    """Copies of the page pools with each request's new token stored at slot
    len_b - 1."""
    k_pages = k_pages.copy()
    v_pages = v_pages.copy()
    ps = k_pages.shape[2]
    for b, L in enumerate(np.asarray(seq_lens).tolist()):
        pos = L - 1
        page = int(block_table[b][pos // ps])
        k_pages[page, :, pos % ps, :] = k_codes[b]
        v_pages[page, :, pos % ps, :] = v_codes[b]
    return k_pages, v_pages

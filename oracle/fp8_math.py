"""Oracle for the native-fp8 product mode (test infrastructure).

The pages report FP8 execution of the model they measure and name cache
precision among the settings a result depends on ([ES-lim]); they say
nothing of attention arithmetic in fp8.  The native-fp8 mode is this
library's own design: with an fp8 cache, QK^T and PV take fp8 operands on
the matrix cores instead of converting the cache to bf16.  Two rounding
steps enter, and the oracle treats them differently:

  * q is quantised per (request, q head): s_q = amax_d |q| / 448 and
    q8 = E4M3(clamp(q / s_q, +-448)), round-to-nearest-even, both divisions
    in float32 (s_q = 1 for an all-zero row).  The score then uses
    s_q * decode(q8).  This step is deterministic, so the oracle takes it
    exactly, deciding the codes in the same float32 arithmetic
    (quantize_q_fp8), and attends exactly with the quantised q
    (attention_fp8q).
  * the softmax weights are rounded to E4M3 before PV (p * 2^8, p <= 1,
    round-to-nearest-even) and the normaliser sums the same rounded weights.
    The rounding happens against the running maximum of the chunk being
    processed, so it is not replayed; weight_rounding_bounds bounds its
    effect instead.

Derivation of the bound, for one (request, q head) and output dim d, with
exact weights p_t = exp(s_t - max s) and output o = sum p v / sum p: let
p'_t be the rounded weights.  For E4M3 (3 fraction bits) a value in the
normal range rounds with relative error at most u = 2^-4, and one in the
subnormal range (below 2^-6, i.e. p < 2^-14 after the 2^8 shift) with
absolute error at most 2^-10 / 2^8 = 2^-18.  A weight rounded while the
running maximum was lower is later multiplied by a factor <= 1, which does
not enlarge either error.  Since o' = sum p' v / sum p',

  o' - o = sum_t (p'_t - p_t)(v_t - o) / sum_t p'_t,

so |o' - o| <= [u sum_t p_t |v_t - o| + 2^-18 sum_t |v_t - o|] / ((1 - u) sum_t p_t)
(worst case: every rounding error aligned).  Treating the relative errors
as independent and uniform within +-u (an upper estimate of their spread)
gives the expected size sqrt(u^2/3 sum_t w_t^2 (v_t - o)^2), w = p / sum p.
"""

import numpy as np

from .codec import fp8_decode, fp8_encode, FP8_MAX, bf16_to_f64
from .attention import attention_reference, attention_selected, row_scales, gather_request
from .attention import decode_kv, _kv_head

U_E4M3 = 2.0 ** -4        # largest relative rounding error in the normal range
SUB_ABS = 2.0 ** -18      # largest absolute error of a shifted weight below 2^-14


def quantize_q_fp8(q):
    """q (bf16 bits [B, Hq, D] or float32 values) -> (codes uint8
    [B, Hq, D], s_q float32 [B, Hq]), deciding in float32."""
    q = np.asarray(q)
    q32 = bf16_to_f64(q).astype(np.float32) if q.dtype == np.uint16 else q.astype(np.float32)
    amax = np.abs(q32).max(axis=-1)
    s_q = np.where(amax > 0, amax / np.float32(FP8_MAX), np.float32(1.0)).astype(np.float32)
    x = (q32 / s_q[..., None]).astype(np.float32)
    x = np.clip(x, np.float32(-FP8_MAX), np.float32(FP8_MAX))
    return fp8_encode(x.astype(np.float64)), s_q


def dequantized_q(q):
    """The q the native-fp8 score uses: s_q * decode(q8), float64."""
    codes, s_q = quantize_q_fp8(q)
    return fp8_decode(codes) * s_q.astype(np.float64)[..., None]


def attention_fp8q(q, k_pages, v_pages, block_table, seq_lens, kv_dtype, sm_scale, **kw):
    """Exact attention (float64) with q replaced by its fp8 quantisation."""
    return attention_reference(dequantized_q(q), k_pages, v_pages, block_table, seq_lens,
                               kv_dtype, sm_scale, **kw)


def weight_rounding_bounds(q_eff, k_pages, v_pages, block_table, seq_lens, kv_dtype, sm_scale,
                           pairs, k_scale=1.0, v_scale=1.0, scale_mode="tensor", k_scales=None,
                           v_scales=None):
    """For each selected (b, h): (o [D], worst-case bound [D], expected
    error size [D]) of the fp8 rounding of the softmax weights, from the
    exact weights (see the module docstring).  q_eff: float64 [B, Hq, D]."""
    q_eff = np.asarray(q_eff, dtype=np.float64)
    Hq = q_eff.shape[1]
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
        s = (k @ q_eff[b, h]) * sm_scale
        p = np.exp(s - s.max())
        z = p.sum()
        o = (p @ v) / z
        dev = np.abs(v - o[None, :])                      # [L, D]
        worst = (U_E4M3 * (p @ dev) + SUB_ABS * dev.sum(axis=0)) / ((1.0 - U_E4M3) * z)
        w = p / z
        rms = np.sqrt((U_E4M3 ** 2 / 3.0) * ((w * w) @ (dev * dev)))
        res[(b, h)] = (o, worst, rms)
    return res

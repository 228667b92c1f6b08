"""Oracle for the native-fp8 product mode (test infrastructure).

The pages report FP8 execution of the model they measure and name cache
precision among the settings a result depends on ([ES-lim]); they say
nothing of attention arithmetic in fp8.  The native-fp8 mode is this
library's own design: with an fp8 cache, QK^T and PV take fp8 operands on
the matrix cores instead of converting the cache to bf16.  Two rounding
steps enter, and the oracle treats them differently:

  * q is quantised per (request, q head): s_q = amax_d |q| / 448,
    x = clamp(q / s_q, +-448), both divisions in float32 (s_q = 1 for an
    all-zero row), as a high part hi = E4M3(x) and a residual
    lo = E4M3(16 (x - decode(hi))), both round-to-nearest-even (the
    difference x - decode(hi) is exact in float32).  The score then uses
    s_q * (decode(hi) + decode(lo) / 16).  The split follows the pages'
    Router GEMM, which keeps an fp32 weight as a high part plus a residual
    stored with a scale and removes the scale in the product (remio.ai
    page, Router GEMM section; arex-research page, Router GEMM paragraph):
    the residual takes q's E4M3 rounding error (relative 2^-4) down to
    about 2^-8.  This step is deterministic, so the oracle takes it exactly,
    deciding the codes in the same float32 arithmetic (quantize_q_fp8,
    quantize_q_residual), and attends exactly with the quantised q
    (attention_fp8q).
  * the softmax weights enter PV in fp8 as well: z = p * 2^8 (p <= 1) is
    kept as a = E4M3(z) plus b = E4M3(z - a), both round-to-nearest-even,
    and PV and the normaliser take a + b (two products into one
    accumulator: the residual split again).  The rounding happens against
    the running maximum of the chunk being processed, so it is not
    replayed; weight_rounding_bounds bounds its effect instead.

Derivation of the bound, for one (request, q head) and output dim d, with
exact weights p_t = exp(s_t - max s) and output o = sum p v / sum p: let
p'_t be the weights PV uses.  E4M3 (3 fraction bits) rounds a value in its
normal range with relative error at most 2^-4 and one in the subnormal
range (below 2^-6) with absolute error at most 2^-10.  So |z - a| <= 2^-4 z
for z >= 2^-6, and b rounds that residual again: |z - a - b| <= 2^-8 z +
2^-10 (also when z or the residual is subnormal), i.e. in weight units
relative error at most u = 2^-8 plus absolute error at most
2^-10 / 2^8 = 2^-18.  A weight rounded while the running maximum was lower
is later multiplied by a factor <= 1, which does not enlarge either error.
Since o' = sum p' v / sum p',

  o' - o = sum_t (p'_t - p_t)(v_t - o) / sum_t p'_t,

so |o' - o| <= [u sum_t p_t |v_t - o| + 2^-18 sum_t |v_t - o|] / ((1 - u) sum_t p_t)
(worst case: every rounding error aligned).  Treating the relative errors
as independent and uniform within +-u (an upper estimate of their spread)
gives the expected size sqrt(u^2/3 sum_t w_t^2 (v_t - o)^2), w = p / sum p.

The arithmetic that evaluates the method adds errors of its own, which the
bound can include (weight_rounding_bounds' score_eps and sum_eps; zero for
the method alone): a score computed with error at most
e_t = score_eps * sm_scale * sum_d |q_d k_td| perturbs its weight by a
factor within exp(+-e_t), i.e. relative error expm1(e_t), added to u for
that token; and the two sums over tokens, each within sum_eps of the sum of
its terms' magnitudes, move o by at most sum_eps (sum_t w_t |v_t| + |o|).
"""

import numpy as np

from .codec import fp8_decode, fp8_encode, FP8_MAX, bf16_to_f64
from .attention import attention_reference, attention_selected, row_scales, gather_request
from .attention import decode_kv, _kv_head

U_E4M3 = 2.0 ** -4        # largest relative rounding error of E4M3 in its normal range
U_WEIGHTS = U_E4M3 ** 2   # largest relative error of a weight kept as value + residual
SUB_ABS = 2.0 ** -18      # largest absolute error of a weight (subnormal floor / 2^8)


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


RESIDUAL_SCALE = 16.0     # the residual is stored x 16 and scaled back by 1/16


def quantize_q_residual(q):
    """The residual codes of q's quantisation: uint8 [B, Hq, D],
    E4M3(16 (x - decode(hi))) with x = clamp(q / s_q) and hi the codes of
    quantize_q_fp8 (the difference taken exactly, as float32 does)."""
    q = np.asarray(q)
    q32 = bf16_to_f64(q).astype(np.float32) if q.dtype == np.uint16 else q.astype(np.float32)
    hi, s_q = quantize_q_fp8(q)
    x = np.clip((q32 / s_q[..., None]).astype(np.float32), np.float32(-FP8_MAX),
                np.float32(FP8_MAX)).astype(np.float64)
    return fp8_encode(RESIDUAL_SCALE * (x - fp8_decode(hi)))


def dequantized_q(q):
    """The q the native-fp8 score uses: s_q * (decode(hi) + decode(lo) / 16),
    float64."""
    hi, s_q = quantize_q_fp8(q)
    lo = quantize_q_residual(q)
    return (fp8_decode(hi) + fp8_decode(lo) / RESIDUAL_SCALE) * s_q.astype(np.float64)[..., None]


def attention_fp8q(q, k_pages, v_pages, block_table, seq_lens, kv_dtype, sm_scale, **kw):
    """Exact attention (float64) with q replaced by its fp8 quantisation."""
    return attention_reference(dequantized_q(q), k_pages, v_pages, block_table, seq_lens,
                               kv_dtype, sm_scale, **kw)


def weight_rounding_bounds(q_eff, k_pages, v_pages, block_table, seq_lens, kv_dtype, sm_scale,
                           pairs, k_scale=1.0, v_scale=1.0, scale_mode="tensor", k_scales=None,
                           v_scales=None, score_eps=0.0, sum_eps=0.0):
    """For each selected (b, h): (o [D], worst-case bound [D], expected
    error size [D]) of the fp8 rounding of the softmax weights, from the
    exact weights (see the module docstring), plus, when score_eps or
    sum_eps is given, the accumulation errors of the arithmetic that
    evaluates it.  q_eff: float64 [B, Hq, D]."""
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
        # relative error of each weight: the rounding's, plus the score's
        u = U_WEIGHTS + np.expm1(score_eps * sm_scale * (np.abs(k) @ np.abs(q_eff[b, h])))
        w = p / z
        sums = sum_eps * (w @ np.abs(v) + np.abs(o))       # [D]
        worst = ((u * p) @ dev + SUB_ABS * dev.sum(axis=0)) / ((1.0 - u.max()) * z) + sums
        rms = np.sqrt(((u * u / 3.0) * w * w) @ (dev * dev) + sums * sums / 3.0)
        res[(b, h)] = (o, worst, rms)
    return res

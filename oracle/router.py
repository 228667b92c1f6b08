"""Oracle for the Router GEMM (test infrastructure).

The router multiplies low-precision activations by fp32 weights whose small
differences can change which experts a token goes to; the operator keeps the
fp32 weights as two bf16 parts, the high part and a residual stored with a
scale (the project documents 1/256), runs two bf16 matrix products in one
kernel and combines them ("Tencent HPC llega a SGLang ...", section on the
Router GEMM; the arex-research page's Router GEMM paragraph: split into two
bf16 components, fused in one kernel, scale correction after the fusion).

Readings taken:
  * activations x are bf16 [T][H]; weights w are fp32 [E][H]; the output is
    the fp32 logits [T][E] = x w^T (the router's score per token and expert);
  * hi = bf16(w) rounded to nearest even; lo = bf16((w - hi) * 256), also
    round-to-nearest-even (w - hi is exact in float32, and so is the product
    by 256, so both sides decide the codes identically); the product is
    x hi^T + (x lo^T) / 256 -- the 1/256 undoes the stored residual's scale;
  * the target is the fp32-weight product: router_reference computes it
    exactly (float64); router_split_reference computes exactly what the split
    represents, x (hi + lo/256)^T.
"""

import numpy as np

from .codec import bf16_to_f64
from .prologue import bf16_encode

RESIDUAL_SCALE = 256.0


def split_router_weights(w):
    """fp32 weights -> (hi, lo) bf16 bit patterns by the rule above."""
    w = np.asarray(w, dtype=np.float32).astype(np.float64)
    hi = bf16_encode(w)
    lo = bf16_encode((w - bf16_to_f64(hi)) * RESIDUAL_SCALE)
    return hi, lo


def split_value(hi, lo):
    """The weight the split represents, float64."""
    return bf16_to_f64(hi) + bf16_to_f64(lo) / RESIDUAL_SCALE


def router_reference(x, w):
    """Exact logits x w^T (float64) from bf16 x bits [T][H] and fp32 w [E][H]."""
    return bf16_to_f64(x) @ np.asarray(w, dtype=np.float32).astype(np.float64).T


def router_split_reference(x, hi, lo):
    """Exact x (hi + lo/256)^T, float64."""
    return bf16_to_f64(x) @ split_value(hi, lo).T


def accumulation_bound(x, hi, lo):
    """A bound on float32 accumulation error of the two products in any
    order: each of the H additions of a sum of |terms| <= S rounds by at most
    one unit of 2^-24 relative to the running magnitude, so the error of one
    product is <= H 2^-24 sum_h |x_h||w_h| (kept loose: 2^-23), and the
    final x hi + x lo / 256 adds one more rounding."""
    ax = np.abs(bf16_to_f64(x))
    H = ax.shape[1]
    mag = ax @ (np.abs(bf16_to_f64(hi)) + np.abs(bf16_to_f64(lo)) / RESIDUAL_SCALE).T
    return H * 2.0 ** -23 * mag + 2.0 ** -23 * np.abs(router_split_reference(x, hi, lo))

"""fp64 CPU oracle for dynamic split-KV paged decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it.  It shares no code with the HIP library; the two meet
only on the byte arrays that the seeded input generators produce.

Everything here is plain numpy in float64 (pure-Python loops only in the
brute-force checker), written for a reader to check against the pages by eye.

Citation keys used in this package (the pages are web articles, cited by
title and section):

  [ES-why]  "Tencent HPC llega a SGLang y desafía a los kernels de inferencia
            predeterminados" (remio.ai), section "Por qué Tencent HPC importa
            para el serving de modelos en línea".  The Polish and Korean pages
            are translations of the same article.
  [ES-lim]  same page, section "Lo que la afirmación de un 48,8 % de TPOT no
            demuestra".
  [ZH-da]   "腾讯混元三算子杀入 SGLang，Hy3 推理延迟暴降 48.8%" (arex-research.com),
            the Dynamic Attention paragraphs printed under the heading
            "Router GEMM：精度不丢，速度翻三倍".
  [EN-vllm] "vLLM × HPC-Ops: High-Performance Attention and MoE Backends from
            Tencent Hunyuan" (8sync news summary), its summary paragraph.

Where the pages leave a step open, the reading taken is named at the function
that implements it.

Parity status: every function in this package is pinned by a CPU test against
something other than itself (brute force, closed forms, library routines,
hand-worked examples); none is "parity unpinned".
"""

from .codec import bf16_to_f64, fp8_decode, fp8_encode, FP8_MAX
from .planner import plan_dynamic, plan_static, Plan
from .attention import (
    gather_request,
    attention_reference,
    attention_selected,
    attention_bruteforce,
    split_merge_reference,
    decode_kv,
    row_scales,
    SCALE_MODES,
)
from .prologue import (rms_norm, rope, prologue_step, bf16_encode, write_new_token,
                       slot_scales)
from .fp8_math import (quantize_q_fp8, quantize_q_residual, dequantized_q, attention_fp8q,
                       weight_rounding_bounds)
from .prefill import prefill_reference, prefill_rows, q_offsets
from .router import (split_router_weights, split_value, router_reference,
                     router_split_reference, accumulation_bound)

__all__ = [
    "bf16_to_f64", "fp8_decode", "fp8_encode", "FP8_MAX",
    "plan_dynamic", "plan_static", "Plan",
    "gather_request", "attention_reference", "attention_selected",
    "attention_bruteforce", "split_merge_reference", "decode_kv", "row_scales",
    "SCALE_MODES", "rms_norm", "rope", "prologue_step", "bf16_encode", "write_new_token",
    "slot_scales", "quantize_q_fp8", "quantize_q_residual", "dequantized_q", "attention_fp8q",
    "weight_rounding_bounds", "prefill_reference", "prefill_rows", "q_offsets",
    "split_router_weights", "split_value", "router_reference", "router_split_reference",
    "accumulation_bound",
]

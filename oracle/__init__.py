"""CPU oracle for the 4-bit routed mixture-of-experts expert layer.

TEST INFRASTRUCTURE ONLY. This package is the plain, slow, obviously correct
definition of what the layer computes, written with numpy on the host. Only the
test suite, the smoke check in ``__graft_entry__`` and the ``cpu_baseline`` leg
of ``bench.py`` may import or run it. The library in ``bit_mixture_experts_amd``
never imports it, and the two share no code, tables or constants.

Sources (web pages, cited by title and section):

* [MXFP4 page] "How do I train and serve MoE models released in MXFP4
  (gpt-oss, DeepSeek-V4)?" -- sections "Two fidelity paths", "Why it happens",
  "Which project solves it", "Supported scope", "Limitations".
* [Solutions index] "MoE Training & Inference Guides -- Cerin Amroth", the
  "Solutions -- one page per problem" tables (grouped-nf4-gemm and
  experts4bit-qlora entries).
* [experts4bit-qlora page] project page "experts4bit-qlora" -- sections
  "What it does", "Use this when", "Limitations -- qlora-fused-moe-experts",
  "Current measured position".
* [Offload page] "How do I offload MoE experts to host RAM, or serve and train
  them from an NVMe arena?" -- section "Why it happens".

Precision: the oracle computes in float64 except where the method itself fixes a
precision: fp32 absmax and the fp32 division that decides an NF4 code; fp32
router logits; and bf16 wherever the layer hands a value to a bf16 GEMM operand
(the model dtype is bf16, accumulation fp32): the dequantised weight
bf16(fp32(level * absmax)), the activation h, the LoRA intermediates xa and
t = dGU B, dGU, and the row-scaled gradient bf16(fp32(w * dOut)). Sums and
outputs (gu, y, out, dX, dA, dB) stay float64. ``layer_forward`` and
``layer_backward`` take exact=True to drop every bf16 step, which the
finite-difference pins of the backward use.

Pin status: every public function has a pin in ``tests/test_oracle_*.py`` that
does not re-use the oracle's own formula (closed forms, exhaustive enumeration,
brute force on tiny inputs, float64 finite differences, torch CPU autograd, the
published NF4 construction). No function is "parity unpinned".
"""

from .numerics import (bf16_bits_from_f32, bf16_bits_to_f64, bf16_bits_to_f32, bf16_round_f64,
                       bf16_other_neighbour_f64)
from .formats import (NF4_LEVELS, nf4_midpoints, quantize_nf4, dequantize_nf4,
                      dequantize_nf4_bf16, E2M1_MAGNITUDES, mxfp4_values, decode_mxfp4_bf16,
                      convert_mxfp4_to_nf4, dq_midpoints, compress_absmax, expand_absmax)
from .routing import route, permute, gather_rows
from .router import (router_logits, router_logits_error_bound, routing_weight_grad,
                     routing_logit_grad)
from .layer import (ExpertWeights, gate_up, activation, down, combine,
                    layer_forward, layer_backward, token_forward)

__all__ = [
    "bf16_bits_from_f32", "bf16_bits_to_f64", "bf16_bits_to_f32", "bf16_round_f64",
    "bf16_other_neighbour_f64",
    "NF4_LEVELS", "nf4_midpoints", "quantize_nf4", "dequantize_nf4", "dequantize_nf4_bf16",
    "E2M1_MAGNITUDES", "mxfp4_values", "decode_mxfp4_bf16", "convert_mxfp4_to_nf4",
    "dq_midpoints", "compress_absmax", "expand_absmax",
    "route", "permute", "gather_rows",
    "router_logits", "router_logits_error_bound", "routing_weight_grad", "routing_logit_grad",
    "ExpertWeights", "gate_up", "activation", "down", "combine",
    "layer_forward", "layer_backward", "token_forward",
]

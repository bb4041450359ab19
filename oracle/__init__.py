"""CPU oracle of the speculative-decoding verifier step -- TEST INFRASTRUCTURE.

This package is the slow, plain reference that the HIP library is checked
against.  It is *not* part of the product: only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call it.  It shares no code with the HIP path (no kernels, headers,
helpers, tables or constants); both sides only share the seeded input
generators in ``synth``.

What it computes, and from where (page titles of the sources):

* two-bit block dequantisation and the eight-bit block dequantisation
  (``formats``) -- the block formats named for the routed-expert and output-head
  weights in the *ds4-on-spark* README (model bullet of its introduction);
  field layout, rounding and nibble order are the readings listed in the design
  notes (the pages name the formats only);
* products, SwiGLU, top-k routing, MoE combine and the vocabulary head
  (``linalg``) -- written as their plain definitions in fp64;
* the p/q accept/reject rule with residual resampling and the bonus token
  (``accept``) -- *Optimizing DeepSeek-V4-Flash on a single NVIDIA GB10/GX10
  with DSpark speculative decoding*, post 1 (the paragraph under the analyzer
  output), taken step by step; target-sample matching -- *1x Spark tuned
  DSpark for DeepSeek-V4-Flash*, the losslessness paragraph; the yield-quench
  accounting -- *ds4-on-spark* README, "The break-even law".

Parity pins (tests marked ``not gpu``) tie every function to facts that do not
come from this code: hand-computed blocks, exact rational arithmetic, closed
forms, brute force and exact enumeration of the emitted-token distribution.
"""
from .formats import (q2_fields, q2_dequant_units, q2_dequant_f32, q2_dequant_f64,
                      q8_fields, q8_dequant_f32, q8_dequant_f64, q2_matrix_bytes,
                      q8_matrix_bytes)
from .linalg import (gemm, silu, swiglu_expert, route_topk, moe_layer, plain_layer,
                     lm_head_logits)
from .accept import (softmax_t, greedy_onehot, distribution, first_exceeding, accept_sequence,
                     spec_accept, target_sample_sequence, spec_accept_target_sample,
                     yield_quench)

__all__ = [
    "q2_fields", "q2_dequant_units", "q2_dequant_f32", "q2_dequant_f64",
    "q8_fields", "q8_dequant_f32", "q8_dequant_f64", "q2_matrix_bytes", "q8_matrix_bytes",
    "gemm", "silu", "swiglu_expert", "route_topk", "moe_layer", "plain_layer",
    "lm_head_logits", "softmax_t", "greedy_onehot", "distribution", "first_exceeding", "accept_sequence", "spec_accept",
    "target_sample_sequence", "spec_accept_target_sample", "yield_quench",
]

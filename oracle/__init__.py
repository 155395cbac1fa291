"""CPU oracle for fused-softmax attention with MX operands.

TEST INFRASTRUCTURE ONLY.  Nothing in the product library imports, links or
calls this package; only the tests, the smoke check and the CPU-baseline leg
of the benchmark do.  It is plain, slow, float64 numpy written to be read
against its sources:

* the pages it follows --
  "Fused-Softmax for efficient quantized attention" (summary paragraph),
  "Moving softmax to matrix operations speeds up AI inference by over 2x"
  (sections "Read it as" and "How it works", with its before/after figure),
  "EFQ-Softmax: Exp-Free Quantization for Softmax" (abstract);
* the OCP Microscaling Formats (MX) v1.0 specification for the element and
  scale encodings, which the pages name by format (MX FP8, FP6 and FP4)
  without defining.

Where the pages leave a step open the oracle takes one plain reading and
says so in the docstring of the function that implements it.

Pin status: every function here is checked by tests that do not re-type its
formulas (brute-force searches, closed forms, special cases, bounds).  The
frozen-max guess has no numeric anchor on the pages and is pinned only by a
hand-worked example of its own definition.
"""

from .mx import (FORMATS, Format, decode, encode_values, round_to_format,
                 mx_quantize, mx_dequantize, pack_codes, unpack_codes,
                 bf16_round)
from .attention import (exact_attention, plain_mx_attention, fused_attention,
                        frozen_max, fused_probabilities, rel_l2)

__all__ = [
    "FORMATS", "Format", "decode", "encode_values", "round_to_format",
    "mx_quantize", "mx_dequantize", "pack_codes", "unpack_codes", "bf16_round",
    "exact_attention", "plain_mx_attention", "fused_attention", "frozen_max",
    "fused_probabilities", "rel_l2",
]

"""CPU oracle for the fused LM-head projection + exact top-k.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this package:
only the tests, the smoke check and the benchmark's CPU-baseline leg do.  It
shares no code with the HIP library or its Python binding.

What it is: the plain definition of what the method computes, written out in
NumPy float64 (lm-head-topk page, intro and section "Method"): form every
logit of the vocabulary projection, then take the k largest under the total
order (value descending, lower vocabulary index first on ties) with a stable
sort.  No chunking, no selection algorithm, no fusion: the method's chunked
select-and-merge reaches exactly this result, so the definition is the oracle.

Modules
  projection  -- dense and binary (dequantized) projection in float64, bf16
                 widening.
  select      -- stable top-k and a sort-free certificate of a top-k result.
  packing     -- logical sign/scale packing of a dense head, and this
                 library's packed byte layout (version 1) written and read by
                 the oracle's own code from the layout's specification.
  normalizer  -- log-sum-exp of each row (the normalizer of the top-k
                 log-probabilities).
  mask        -- a grammar bitmask applied to logits (disallowed -> -inf).
  sample      -- one token drawn from the top-k survivors: temperature, the
                 top-k / top-p / min-p keep set, a Gumbel-max draw from a
                 Philox4x32-10 counter-based generator.
"""

from .projection import (
    bf16_bits_to_f32,
    project_binary,
    project_dense,
)
from .select import certify_topk, float_key_order, topk_stable, topk_stable_rows
from .normalizer import logsumexp_row, logsumexp_rows
from .mask import allowed_bool, apply_allowed
from .sample import (
    draw_uniform,
    gumbel,
    keep_count,
    philox4x32_10,
    sample_row,
    sample_rows,
    uniform_from_word,
)
from .packing import (
    pack_layout_bytes,
    pack_logical,
    packed_sizes,
    unpack_layout_bytes,
)

__all__ = [
    "bf16_bits_to_f32",
    "project_binary",
    "project_dense",
    "certify_topk",
    "float_key_order",
    "logsumexp_row",
    "allowed_bool",
    "apply_allowed",
    "logsumexp_rows",
    "topk_stable",
    "topk_stable_rows",
    "pack_layout_bytes",
    "pack_logical",
    "packed_sizes",
    "unpack_layout_bytes",
    "philox4x32_10",
    "uniform_from_word",
    "draw_uniform",
    "gumbel",
    "keep_count",
    "sample_row",
    "sample_rows",
]

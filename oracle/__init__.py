"""CPU fp64 oracle for exact attention.

TEST INFRASTRUCTURE ONLY. The attention library never imports, calls or links
anything in this package; only the test suite, the smoke check and the bench's
CPU-baseline leg use it. It shares no code with the HIP path.

* ``attention``: the plain definition, softmax(scale * q k^T) v, with the full
  score matrix materialised in float64, its row logsumexp, and the gradients
  obtained from the calculus of that definition.
* ``blocksparse``: the definition restricted to the (query block, key block)
  pairs a block mask enables, in float64.
* ``fp8``: e4m3 codes from their bit fields, block-wise quantisation with one
  float32 scale per 64 rows, and the definition on the dequantised inputs.
* ``online``: the tiled online-softmax recurrence in its two published forms
  (normalise every block; defer the normalisation to the end), in float64,
  written from the pages' description. It exists to check that tiling reaches
  the same result as the definition.

Parity status: every function here is pinned by tests under ``-m "not gpu"``
against closed forms, hand-derived worked examples, identities, brute-force
finite differences and a library routine (torch CPU float64).
"""
from .attention import (
    attention_fwd,
    attention_fwd_rows,
    attention_probs,
    attention_bwd,
    attention_bwd_head,
    causal_tile_count,
)
from .blocksparse import attention_fwd_blockmask, element_mask
from .fp8 import (
    E4M3_MAX,
    attention_fwd_fp8,
    dequantize_blockwise_e4m3,
    e4m3_decode,
    e4m3_encode,
    e4m3_values,
    quantize_blockwise_e4m3,
)
from .online import online_fwd_normalise_each_block, online_fwd_deferred

__all__ = [
    "attention_fwd",
    "attention_fwd_rows",
    "attention_probs",
    "attention_bwd",
    "attention_bwd_head",
    "causal_tile_count",
    "attention_fwd_blockmask",
    "element_mask",
    "E4M3_MAX",
    "attention_fwd_fp8",
    "dequantize_blockwise_e4m3",
    "e4m3_decode",
    "e4m3_encode",
    "e4m3_values",
    "quantize_blockwise_e4m3",
    "online_fwd_normalise_each_block",
    "online_fwd_deferred",
]

"""Oracle for exact scaled-dot-product attention -- TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, float64 CPU statement of what the attention
forward computes, written from the source pages:

* "Attention and Its Computational Cost" (programmer.ie inference book,
  chapter 8), section "What is being computed": two matrix products and a
  softmax per head; S and P are both T_q x T_kv.
* "FlashAttention IO-aware tiling lab" (parsercheat.com), the caption
  S = QK^T / sqrt(d), P = softmax(S), O = PV.
* "IO-Aware Attention: Tiling the Score Matrix Without Materializing It"
  (mercemay.com), section "Softmax over blocks, exactly" (the running max /
  running sum recurrence) and section "Parallelism and the cost of the split"
  (partial outputs over key partitions merged with the same rescaling).
* "E8.1 IO-aware attention" (coursefy.online), the worked example and the
  "Do it in code" function specs.
* Backward (``backward.py``): "IO-Aware Attention", section "What has to stay
  in fast memory" -- P is recomputed from Q, K, V and the saved row constants;
  the gradient formulas are the calculus of the forward definition.

Who may use it: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``.  The product package
(``io_aware_exact_amd``) never imports, calls or links anything here, and
nothing here imports the product package.  The oracle shares no code, tables
or constants with the HIP path.

Parity status: every public function is pinned by ``tests/test_oracle.py``,
``tests/test_oracle_backward.py`` and ``tests/test_cost_model.py`` against values printed on the pages
(``tests/golden/``), closed forms, special cases, brute force on tiny inputs
and a library routine; none is "parity unpinned".
"""

from .attention import (
    attention,
    attention_gqa,
    combine_partials,
    online_attention,
    online_softmax_states,
    split_attention,
    standard_attention,
)
from .backward import attention_backward, attention_backward_from_lse
from .cost import (
    attention_flops,
    causal_pairs,
    fit_exponent,
    kv_bytes,
    min_transfer_time,
    num_blocks,
    score_bytes,
    score_tensor_bytes,
    tile_bytes,
)

__all__ = [
    "attention",
    "attention_backward",
    "attention_backward_from_lse",
    "attention_gqa",
    "combine_partials",
    "online_attention",
    "online_softmax_states",
    "split_attention",
    "standard_attention",
    "attention_flops",
    "causal_pairs",
    "fit_exponent",
    "kv_bytes",
    "min_transfer_time",
    "num_blocks",
    "score_bytes",
    "score_tensor_bytes",
    "tile_bytes",
]

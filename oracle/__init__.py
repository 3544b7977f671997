"""fp64 CPU oracle for streaming attention -- TEST INFRASTRUCTURE ONLY.

This package is the checker, not the product.  Only the test suite, the smoke
check in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import
it.  The GPU library never calls into it, and it shares no code, constants or
helpers with the GPU library: it receives plain numpy arrays and computes the
attention result straight from its definition, in float64.

Sources (the pages the method is described on):
  * "ADR-0060: AHBM GQA Fused Attention kernel (Llama3-70B)" -- the per-tile
    online-softmax sequence (its section 3), the log-sum-exp merge of partial
    results (section 4), GQA M-fold (section 5.2), the causal tile classes
    (section 5.4), the kernel I/O contract (section 0.5).
  * "AttentionRegion Transformation -- Deriving FlashAttention via
    Memory-Centric Compilation in AICF" -- the score and probability matrices
    are not materialised (section 5), the online-softmax recurrence (section 6).
  * "AI Compiler pipeline stages" (teach-meaning 1601) -- the canonical stable
    softmax form and the causal attention pattern.

Every function is pinned by CPU tests (``tests/test_oracle_*.py``) against
brute force, closed forms and invariants; see each function's docstring.
"""

from .attn_f64 import (  # noqa: F401
    attention,
    attention_rows,
    attention_online,
    partial_attention,
    attention_key_range,
    merge_partials,
    decode_attention,
    paged_attention,
    visible_keys,
)

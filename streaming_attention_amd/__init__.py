"""Streaming attention forward for AMD Instinct MI355X (gfx950).

Fused prefill (GQA, causal; split-KV for short query blocks after a long
prefix), split-KV decode, multi-token decode over a paged KV cache and the
log-sum-exp combine, as
hand-written HIP kernels behind the C ABI in ``include/attn.h``.  This package
is the thin Python binding over ``libattn.so`` plus the seeded workloads.
"""

from ._binding import (  # noqa: F401
    AttnError,
    LIB_PATH,
    combine_lse,
    decode,
    decode_paged,
    decode_splitkv,
    lib,
    paged_splits,
    prefill,
    prefill_splits,
    prefill_splitkv,
    splits_for_lengths,
)
from . import workloads  # noqa: F401

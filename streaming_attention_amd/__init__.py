"""Streaming attention forward for AMD Instinct MI355X (gfx950).

Fused prefill (GQA, causal; split-KV for short query blocks after a long
prefix), split-KV decode, multi-token decode over a paged KV cache and the
log-sum-exp combine, as
hand-written HIP kernels behind the C ABI in ``include/attn.h``.  This package
is the thin Python binding over ``libattn.so``, the seeded workloads, and
``sdpa_frontend``, a torch.fx pass that routes attention written in PyTorch to
the fused kernel.
"""

from ._binding import (  # noqa: F401
    AttnError,
    LIB_PATH,
    combine_lse,
    decode,
    decode_noalloc,
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
from . import sdpa_frontend  # noqa: F401

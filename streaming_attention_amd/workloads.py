"""Seeded synthetic workloads: the problem shapes the library is measured and
checked on, and the generators that fill them.

This module holds only shapes, seeds and random-number recipes -- none of the
attention arithmetic.  The tests, the bench and the smoke check draw inputs
here and hand the same tensors to both the GPU library and the float64 oracle.

Recipe (every workload): ``g = torch.Generator(device).manual_seed(seed)``,
then draw Q, K, V in that order with ``torch.randn(..., dtype=float32,
generator=g)`` and cast to the storage dtype (bf16 unless the workload says
fp32).  Ragged decode lengths come first, from their own CPU generator with
the same seed: ``torch.randint(lo, hi + 1, (B,))``.  The values depend on the
device the generator runs on; both sides of a check always see the same
tensor.  Layout ``[B, H, S, d]``
contiguous.  The Llama3-70B head geometry (64 query heads, 8 KV heads, d=128)
is the one of "ADR-0060: AHBM GQA Fused Attention kernel", section 0.
"""

from __future__ import annotations

import dataclasses
import math

import torch


@dataclasses.dataclass(frozen=True)
class Prefill:
    name: str
    B: int
    Hq: int
    Hkv: int
    Sq: int
    Skv: int
    d: int
    dtype: str          # "bf16" or "f32"
    causal: bool
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def visible_pairs_per_head(self) -> int:
        """Number of (query, key) pairs a query head attends over."""
        if not self.causal:
            return self.Sq * self.Skv
        q_start = self.Skv - self.Sq
        # row t sees keys 0 .. q_start + t  ->  q_start + t + 1 keys
        return self.Sq * (q_start + 1) + self.Sq * (self.Sq - 1) // 2

    def flops(self) -> int:
        """Algorithmic FLOPs of the two GEMMs on visible pairs: 4 * d * pairs."""
        return 4 * self.d * self.B * self.Hq * self.visible_pairs_per_head()


@dataclasses.dataclass(frozen=True)
class Decode:
    name: str
    B: int
    Hq: int
    Hkv: int
    S_cap: int
    d: int
    seed: int
    fixed_len: int | None        # every sequence this long (None: ragged draw)
    len_lo: int = 0              # ragged: lengths uniform in [len_lo, len_hi]
    len_hi: int = 0
    splits: int | None = None    # fixed split count (None: chosen per length)
    nan_padding: bool = False    # fill cache slots beyond each length with NaN
    dtype: str = "bf16"

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32


@dataclasses.dataclass(frozen=True)
class PagedDecode:
    """T_q new tokens per sequence over a paged KV cache (pages of 64
    positions, shuffled in the pool), ragged lengths uniform in [len_lo, len_hi]."""
    name: str
    B: int
    Hq: int
    Hkv: int
    T_q: int
    d: int
    seed: int
    len_lo: int
    len_hi: int
    spare_pages: int = 8          # pool pages no sequence uses (NaN-filled)
    page: int = 64
    dtype: str = "bf16"

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32


# The workloads, smallest first.
SINGLE_HEAD_F32 = Prefill("single_head_f32_s128_d64", B=1, Hq=1, Hkv=1, Sq=128, Skv=128,
                          d=64, dtype="f32", causal=False, seed=1)
MHA_CAUSAL = Prefill("mha_causal_b2_h16_s1024_d64", B=2, Hq=16, Hkv=16, Sq=1024, Skv=1024,
                     d=64, dtype="bf16", causal=True, seed=2)
GQA70B_PREFILL = Prefill("gqa70b_causal_prefill_b1_s8192", B=1, Hq=64, Hkv=8, Sq=8192,
                         Skv=8192, d=128, dtype="bf16", causal=True, seed=3)
GQA70B_DECODE = Decode("gqa70b_decode_b4_kv32768_64splits", B=4, Hq=64, Hkv=8, S_cap=32768,
                       d=128, seed=4, fixed_len=32768, splits=64)
RAGGED_DECODE = Decode("ragged_decode_b16_len1k_128k", B=16, Hq=64, Hkv=8, S_cap=131072,
                       d=128, seed=5, fixed_len=None, len_lo=1024, len_hi=131072,
                       splits=None, nan_padding=True)
CHUNKED_PREFILL = Prefill("chunked_prefill_q512_prefix65536", B=1, Hq=64, Hkv=8, Sq=512,
                          Skv=65536 + 512, d=128, dtype="bf16", causal=True, seed=6)

PAGED_DECODE = PagedDecode("paged_decode_b16_tq4_len1k_32k", B=16, Hq=64, Hkv=8, T_q=4, d=128, seed=7,
                           len_lo=1024, len_hi=32768)

PREFILL_WORKLOADS = [SINGLE_HEAD_F32, MHA_CAUSAL, GQA70B_PREFILL, CHUNKED_PREFILL]
DECODE_WORKLOADS = [GQA70B_DECODE, RAGGED_DECODE]


def _randn(shape, g, device, dtype):
    return torch.randn(shape, dtype=torch.float32, generator=g, device=device).to(dtype)


def prefill_inputs(w: Prefill, device="cpu", *, Sq=None, Skv=None, B=None):
    """Q, K, V for a prefill workload (sizes may be overridden for small cases)."""
    B = w.B if B is None else B
    Sq = w.Sq if Sq is None else Sq
    Skv = w.Skv if Skv is None else Skv
    g = torch.Generator(device=device).manual_seed(w.seed)
    q = _randn((B, w.Hq, Sq, w.d), g, device, w.torch_dtype)
    k = _randn((B, w.Hkv, Skv, w.d), g, device, w.torch_dtype)
    v = _randn((B, w.Hkv, Skv, w.d), g, device, w.torch_dtype)
    return q, k, v


def decode_lengths(w: Decode, B=None) -> torch.Tensor:
    """Per-sequence KV lengths (int32, CPU).  Drawn first from the seed."""
    B = w.B if B is None else B
    if w.fixed_len is not None:
        return torch.full((B,), w.fixed_len, dtype=torch.int32)
    g = torch.Generator(device="cpu").manual_seed(w.seed)
    return torch.randint(w.len_lo, w.len_hi + 1, (B,), generator=g).to(torch.int32)


def decode_inputs(w: Decode, device="cpu", *, B=None, S_cap=None, lengths=None):
    """Q ``[B,Hq,1,d]``, K/V caches ``[B,Hkv,S_cap,d]`` and lengths for decode.

    Lengths come from :func:`decode_lengths` unless given.  K/V are drawn per
    sequence (so that long caches never need one huge fp32 temporary); slots at
    or beyond a sequence's length are NaN when ``nan_padding`` is set, which
    proves that only valid keys are read.
    """
    B = w.B if B is None else B
    S_cap = w.S_cap if S_cap is None else S_cap
    lens = decode_lengths(w, B) if lengths is None else lengths.to(torch.int32).cpu()
    g = torch.Generator(device=device).manual_seed(w.seed)
    q = _randn((B, w.Hq, 1, w.d), g, device, w.torch_dtype)
    k = torch.empty((B, w.Hkv, S_cap, w.d), dtype=w.torch_dtype, device=device)
    v = torch.empty_like(k)
    for b in range(B):
        k[b] = _randn((w.Hkv, S_cap, w.d), g, device, w.torch_dtype)
        v[b] = _randn((w.Hkv, S_cap, w.d), g, device, w.torch_dtype)
        if w.nan_padding:
            n = int(lens[b])
            k[b, :, n:] = float("nan")
            v[b, :, n:] = float("nan")
    return q, k, v, lens


def decode_kv_bytes(lens, Hkv: int, d: int, elem_bytes: int = 2) -> int:
    """Algorithmic KV bytes of one decode step: every valid K and V byte once."""
    return int(sum(int(x) for x in lens)) * Hkv * d * elem_bytes * 2


def paged_lengths(w: PagedDecode, B=None) -> torch.Tensor:
    """Per-sequence KV lengths (int32, CPU), drawn first from the seed."""
    B = w.B if B is None else B
    g = torch.Generator(device="cpu").manual_seed(w.seed)
    return torch.randint(w.len_lo, w.len_hi + 1, (B,), generator=g).to(torch.int32)


def paged_inputs(w: PagedDecode, device="cpu", *, B=None, lengths=None):
    """Q ``[B,Hq,T_q,d]``, page pools ``[num_pages,Hkv,page,d]`` for K and V,
    block table ``[B,max_pages]`` int32 and lengths ``[B]`` int32 (CPU).

    Lengths come first (CPU generator), then the pool placement: a random
    permutation of all pool pages (same CPU generator), consumed in sequence
    order.  Then Q and each sequence's K and V (device generator), written page
    by page to their pool slots.  Positions past a sequence's length in its
    last page, and the spare pages, are NaN; unused block-table entries point
    at a spare page.
    """
    B = w.B if B is None else B
    gc = torch.Generator(device="cpu").manual_seed(w.seed)
    drawn = torch.randint(w.len_lo, w.len_hi + 1, (B,), generator=gc).to(torch.int32)   # = paged_lengths
    lens = drawn if lengths is None else lengths.to(torch.int32).cpu()
    n_pages = [-(-int(n) // w.page) for n in lens]
    max_pages = max(max(n_pages), 1)
    total = sum(n_pages) + w.spare_pages
    order = torch.randperm(total, generator=gc)
    table = torch.full((B, max_pages), int(order[total - 1]), dtype=torch.int32)
    g = torch.Generator(device=device).manual_seed(w.seed)
    q = _randn((B, w.Hq, w.T_q, w.d), g, device, w.torch_dtype)
    kp = torch.full((total, w.Hkv, w.page, w.d), float("nan"), dtype=w.torch_dtype, device=device)
    vp = torch.full_like(kp, float("nan"))
    nxt = 0
    for b in range(B):
        n = int(lens[b])
        kb = _randn((w.Hkv, n_pages[b] * w.page, w.d), g, device, w.torch_dtype)
        vb = _randn((w.Hkv, n_pages[b] * w.page, w.d), g, device, w.torch_dtype)
        kb[:, n:] = float("nan")
        vb[:, n:] = float("nan")
        for p_ in range(n_pages[b]):
            slot = int(order[nxt])
            nxt += 1
            table[b, p_] = slot
            kp[slot] = kb[:, p_ * w.page:(p_ + 1) * w.page]
            vp[slot] = vb[:, p_ * w.page:(p_ + 1) * w.page]
    return q, kp, vp, table, lens

"""attn_decode_noalloc (split partials in the library's fixed workspace) on the
GPU against attn_decode (the same decode with caller-supplied workspace)."""

import math

import pytest
import torch

import streaming_attention_amd as sa
from streaming_attention_amd import workloads as W
from parity import assert_lse, assert_o

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _small_case():
    B, Hq, Hkv, S_cap, d = 3, 8, 1, 700, 128
    g = torch.Generator(device=DEV).manual_seed(555)
    q = torch.randn((B, Hq, 1, d), generator=g, device=DEV).to(torch.bfloat16)
    k = torch.randn((B, Hkv, S_cap, d), generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn((B, Hkv, S_cap, d), generator=g, device=DEV).to(torch.bfloat16)
    lens = [700, 1, 333]
    for b, n in enumerate(lens):           # poison everything past each length
        k[b, :, n:] = float("nan")
        v[b, :, n:] = float("nan")
    lt = torch.tensor(lens, dtype=torch.int32, device=DEV)
    nt = torch.tensor([4, 1, 3], dtype=torch.int32, device=DEV)
    return q, k, v, lt, nt, 4, 1 / math.sqrt(d)


def test_noalloc_decode_matches_attn_decode_on_two_calls():
    """The 70B-shape decode (4 x 64 heads x 64 splits: 16,384 partials), then a
    smaller ragged decode with fewer splits on the same workspace: each output
    against attn_decode's at the bar, and the second is not disturbed by the
    partials the first left behind."""
    w = W.GQA70B_DECODE
    q, k, v, _ = W.decode_inputs(w, DEV)
    small = _small_case()
    cases = [(q, k, v, None, None, w.splits, w.scale), small]
    for i, (qq, kk, vv, lt, nt, ms, scale) in enumerate(cases):
        o_ref, l_ref = sa.decode(qq, kk, vv, lt, nt, max_splits=ms, scale=scale, fused=True)
        o = torch.full_like(o_ref, float("nan"))
        lse = torch.full_like(l_ref, float("nan"))
        sa.decode_noalloc(qq, kk, vv, lt, nt, max_splits=ms, scale=scale, out=o, lse=lse)
        torch.cuda.synchronize()
        assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all(), f"call {i}: output not written"
        assert_o(o.float(), o_ref.float(), "bf16", f"O call {i}")
        assert_lse(lse, l_ref, "bf16", f"LSE call {i}")


def test_noalloc_decode_refuses_more_partials_than_its_workspace():
    q = torch.zeros(16, 64, 1, 128, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros(16, 8, 64, 128, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(sa.AttnError, match="WORKSPACE"):
        sa.decode_noalloc(q, k, k, max_splits=65)          # 16 * 64 * 65 > 65536

"""The C ABI library on the CPU: it loads, exports every function the header
declares, and rejects invalid arguments on the host before any HIP call."""

import ctypes
import os
import re

import pytest
import torch

import streaming_attention_amd as sa
from streaming_attention_amd import _binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

OK, NULL, SHAPE, UNSUP, ALIGN = 0, 1, 2, 3, 4
BF16, F32 = 1, 0
P = 0x10000          # a 16-byte aligned non-null address; never dereferenced here
MIS = 0x10008        # 8-byte aligned only


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_every_entry_point():
    names = declared_functions()
    for n in ("attn_prefill", "attn_prefill_splitkv", "attn_decode_splitkv", "attn_combine_lse", "attn_decode",
              "attn_decode_noalloc", "attn_decode_paged", "attn_status_string"):
        assert n in names


def test_library_loads_and_exports_every_declared_symbol():
    lib = sa.lib()
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in attn.h but not exported"
    assert set(_binding.SIGNATURES) == set(declared_functions())


def test_status_strings():
    lib = sa.lib()
    for code in range(7):
        s = lib.attn_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.attn_status_string(99).decode() == "unknown status"


def prefill(q=P, k=P, v=P, o=P, lse=P, B=1, Hq=8, Hkv=2, Sq=16, Skv=32, d=128, dtype=BF16, causal=1,
            scale=0.088, stream=None):
    return sa.lib().attn_prefill(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, d, dtype, causal, scale, stream)


def prefill_split(q=P, k=P, v=P, po=P, pl=P, B=1, Hq=8, Hkv=2, Sq=16, Skv=32, d=128, n=4, dtype=BF16, causal=1,
                  scale=0.088, stream=None):
    return sa.lib().attn_prefill_splitkv(q, k, v, po, pl, B, Hq, Hkv, Sq, Skv, d, n, dtype, causal, scale, stream)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), NULL), (dict(po=None), NULL), (dict(pl=None), NULL), (dict(k=None), NULL),
    (dict(n=0), SHAPE), (dict(n=257), SHAPE), (dict(Hq=6, Hkv=4), SHAPE), (dict(Sq=40, Skv=32), SHAPE),
    (dict(scale=0.0), SHAPE), (dict(dtype=F32), UNSUP), (dict(d=96), UNSUP), (dict(dtype=5), UNSUP),
    (dict(q=MIS), ALIGN), (dict(po=MIS), ALIGN), (dict(pl=MIS), ALIGN), (dict(v=MIS), ALIGN),
    (dict(B=0), OK), (dict(Sq=0), OK), (dict(B=0, q=None, po=None, pl=None), OK),
    (dict(Hq=64, Hkv=8, Sq=1 << 20, Skv=1 << 20, B=64, n=64), SHAPE),
    (dict(Skv=1 << 23, Sq=16, n=1), UNSUP),   # K/V slice of one KV head >= 2 GiB
])
def test_prefill_splitkv_host_validation(kw, expect):
    assert prefill_split(**kw) == expect


def paged(q=P, kp=P, vp=P, bt=P, kl=P, ns=None, B=2, Hq=8, Hkv=2, T_q=4, num_pages=10, max_pages=4, d=128,
          n=1, dtype=BF16, scale=0.088, po=P, pl=P, o=P, lse=P, stream=None):
    return sa.lib().attn_decode_paged(q, kp, vp, bt, kl, ns, B, Hq, Hkv, T_q, num_pages, max_pages, d, n, dtype,
                                      scale, po, pl, o, lse, stream)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), NULL), (dict(kp=None), NULL), (dict(bt=None), NULL), (dict(kl=None), NULL),
    (dict(o=None), NULL), (dict(n=2, po=None), NULL), (dict(n=2, o=None, lse=None, pl=None), NULL),
    (dict(n=0), SHAPE), (dict(n=300), SHAPE), (dict(Hq=6, Hkv=4), SHAPE), (dict(num_pages=0), SHAPE),
    (dict(max_pages=0), SHAPE), (dict(T_q=-1), SHAPE), (dict(scale=0.0), SHAPE),
    (dict(dtype=F32), UNSUP), (dict(d=80), UNSUP), (dict(max_pages=1 << 26), UNSUP),
    (dict(q=MIS), ALIGN), (dict(kp=MIS), ALIGN), (dict(o=MIS), ALIGN), (dict(n=3, pl=MIS), ALIGN),
    (dict(B=0), OK), (dict(T_q=0), OK), (dict(B=0, q=None, kp=None, bt=None), OK),
])
def test_decode_paged_host_validation(kw, expect):
    assert paged(**kw) == expect


def decode(q=P, k=P, v=P, kv_len=None, ns=None, B=2, Hq=8, Hkv=2, S_cap=100, d=128, max_splits=8,
           dtype=BF16, scale=0.088, po=P, pl=P, stream=None):
    return sa.lib().attn_decode_splitkv(q, k, v, kv_len, ns, B, Hq, Hkv, S_cap, d, max_splits, dtype, scale,
                                        po, pl, stream)


def decode_fused(q=P, k=P, v=P, kv_len=None, ns=None, B=2, Hq=8, Hkv=2, S_cap=100, d=128, max_splits=8,
                 dtype=BF16, scale=0.088, po=P, pl=P, cnt=P, o=P, lse=P, stream=None):
    return sa.lib().attn_decode(q, k, v, kv_len, ns, B, Hq, Hkv, S_cap, d, max_splits, dtype, scale,
                                po, pl, cnt, o, lse, stream)


@pytest.mark.parametrize("kw,expect", [
    (dict(cnt=None), NULL), (dict(o=None), NULL), (dict(q=None), NULL), (dict(po=None), NULL),
    (dict(max_splits=0), SHAPE), (dict(Hq=6, Hkv=4), SHAPE), (dict(scale=-1.0), SHAPE),
    (dict(dtype=F32), UNSUP), (dict(Hq=64, Hkv=2), UNSUP), (dict(cnt=MIS), ALIGN), (dict(o=MIS), ALIGN),
    (dict(B=0), OK), (dict(B=0, cnt=None, o=None), OK),
])
def test_fused_decode_host_validation(kw, expect):
    assert decode_fused(**kw) == expect


def decode_noalloc(q=P, k=P, v=P, kv_len=None, ns=None, B=2, Hq=8, Hkv=2, S_cap=100, d=128, max_splits=8,
                   dtype=BF16, scale=0.088, o=P, lse=P, stream=None):
    return sa.lib().attn_decode_noalloc(q, k, v, kv_len, ns, B, Hq, Hkv, S_cap, d, max_splits, dtype, scale,
                                        o, lse, stream)


WORKSPACE = 6


@pytest.mark.parametrize("kw,expect", [
    (dict(o=None), NULL), (dict(q=None), NULL), (dict(k=None), NULL),
    (dict(max_splits=0), SHAPE), (dict(Hq=6, Hkv=4), SHAPE), (dict(scale=-1.0), SHAPE),
    (dict(dtype=F32), UNSUP), (dict(Hq=64, Hkv=2), UNSUP), (dict(o=MIS), ALIGN), (dict(lse=MIS), ALIGN),
    (dict(B=0), OK), (dict(B=0, o=None, q=None), OK),
    (dict(B=16, Hq=64, Hkv=8, max_splits=65), WORKSPACE),       # 16 * 64 * 65 > 65536 partials
    (dict(B=1 << 12, Hq=16, Hkv=2, max_splits=2), WORKSPACE),
    (dict(B=16, Hq=64, Hkv=8, max_splits=65, o=None), WORKSPACE),   # the size check comes first
])
def test_decode_noalloc_host_validation(kw, expect):
    assert decode_noalloc(**kw) == expect


def combine(po=P, pl=P, ns=None, B=2, Hq=8, max_splits=8, d=128, o=P, lse=P, dtype=BF16, stream=None):
    return sa.lib().attn_combine_lse(po, pl, ns, B, Hq, max_splits, d, o, lse, dtype, stream)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), NULL), (dict(o=None), NULL), (dict(k=None), NULL), (dict(v=None), NULL),
    (dict(Hq=6, Hkv=4), SHAPE), (dict(Hkv=0), SHAPE), (dict(Hq=0), SHAPE), (dict(B=-1), SHAPE),
    (dict(Sq=-3), SHAPE), (dict(Skv=-1), SHAPE), (dict(Sq=40, Skv=32, causal=1), SHAPE),
    (dict(scale=0.0), SHAPE), (dict(scale=-0.5), SHAPE), (dict(scale=float("nan")), SHAPE),
    (dict(scale=float("inf")), SHAPE), (dict(d=96), UNSUP), (dict(d=256), UNSUP), (dict(dtype=7), UNSUP),
    (dict(q=MIS), ALIGN), (dict(k=MIS), ALIGN), (dict(o=MIS), ALIGN), (dict(lse=MIS), ALIGN),
    (dict(B=0), OK), (dict(Sq=0), OK), (dict(B=0, q=None, o=None), OK),
    (dict(Hq=64, Hkv=8, Sq=1 << 28, Skv=1 << 28, B=64), SHAPE),
    (dict(Skv=1 << 23, Sq=16), UNSUP), (dict(Hq=64, Hkv=1, Sq=1 << 17, Skv=1 << 17), UNSUP),
])
def test_prefill_host_validation(kw, expect):
    assert prefill(**kw) == expect


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), NULL), (dict(po=None), NULL), (dict(pl=None), NULL), (dict(k=None), NULL),
    (dict(max_splits=0), SHAPE), (dict(max_splits=257), SHAPE), (dict(Hq=6, Hkv=4), SHAPE),
    (dict(B=-2), SHAPE), (dict(S_cap=-1), SHAPE), (dict(scale=0.0), SHAPE),
    (dict(dtype=F32), UNSUP), (dict(d=80), UNSUP), (dict(Hq=64, Hkv=2), UNSUP),
    (dict(q=MIS), ALIGN), (dict(po=MIS), ALIGN), (dict(v=MIS), ALIGN),
    (dict(B=0), OK), (dict(B=0, q=None, po=None, pl=None), OK),
])
def test_decode_host_validation(kw, expect):
    assert decode(**kw) == expect


@pytest.mark.parametrize("kw,expect", [
    (dict(po=None), NULL), (dict(pl=None), NULL), (dict(o=None), NULL),
    (dict(max_splits=0), SHAPE), (dict(max_splits=300), SHAPE), (dict(Hq=0), SHAPE), (dict(B=-1), SHAPE),
    (dict(d=32), UNSUP), (dict(dtype=9), UNSUP), (dict(o=MIS), ALIGN), (dict(lse=MIS), ALIGN),
    (dict(B=0), OK),
])
def test_combine_host_validation(kw, expect):
    assert combine(**kw) == expect


def test_binding_rejects_cpu_tensors_before_calling_the_library():
    q = torch.zeros(1, 2, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        sa.prefill(q, q[:, :1], q[:, :1])
    with pytest.raises(ValueError):
        sa.decode_splitkv(q[:, :, :1], q, q)


def test_binding_has_no_fallback(monkeypatch, tmp_path):
    """A missing library is an error, not a silent CPU path."""
    monkeypatch.setattr(_binding, "_lib", None)
    monkeypatch.setattr(_binding, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        _binding.lib()


def test_prefill_splits_heuristic():
    assert sa.prefill_splits(1, 64, 8, 512, 66048) == 2        # 128 blocks of 256 rows after a 64K prefix
    assert sa.prefill_splits(1, 64, 8, 8192, 8192) == 1        # 2048 blocks already
    assert sa.prefill_splits(1, 64, 8, 512, 66048, torch.float32) == 1
    assert sa.prefill_splits(1, 8, 8, 64, 1 << 20) == 32       # few rows, long prefix: 8 blocks x 32
    assert sa.prefill_splits(1, 8, 1, 200, 333) == 1           # too few key tiles to split


def test_paged_splits_heuristic():
    assert sa.paged_splits(16, 64, 8, 4, 512) == 6      # 32 stacked rows, 128 (sequence, KV head) pairs -> 6 splits
    assert sa.paged_splits(1, 64, 8, 1, 4096) == 96     # one sequence: split its keys widely
    assert sa.paged_splits(64, 64, 8, 4, 8) == 1        # 512 keys at most: no split
    assert sa.paged_splits(4, 64, 8, 16, 512) == 32     # 128 stacked rows (the prefill kernel's paged mode): 32 blocks -> 1024 / 32


def test_splits_for_lengths():
    n = sa.splits_for_lengths(torch.tensor([0, 1, 2048, 2049, 131072, 10 ** 7]))
    assert n.tolist() == [1, 1, 1, 2, 64, 64]
    assert n.dtype == torch.int32


@pytest.mark.gpu
def test_binding_rejects_output_buffers_of_the_wrong_shape():
    """Caller-supplied outputs and split counts are checked against the shapes
    the kernels write before anything is launched."""
    dev = "cuda"
    bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32
    B, Hq, Hkv, S, d, n = 2, 8, 2, 128, 128, 4
    q = torch.zeros(B, Hq, 1, d, device=dev, dtype=bf)
    kc = torch.zeros(B, Hkv, S, d, device=dev, dtype=bf)
    po = torch.zeros(B, Hq, n, d, device=dev, dtype=f32)
    pl = torch.zeros(B, Hq, n, device=dev, dtype=f32)
    with pytest.raises(ValueError, match="shape"):
        sa.combine_lse(po, pl, torch.ones(B + 1, device=dev, dtype=i32))
    with pytest.raises(ValueError, match="shape"):
        sa.combine_lse(po, pl, None, bf, out=torch.zeros(B, Hq - 1, 1, d, device=dev, dtype=bf))
    with pytest.raises(ValueError, match="shape"):
        sa.combine_lse(po, pl, None, bf, lse=torch.zeros(B, 1, device=dev, dtype=f32))
    with pytest.raises(ValueError, match="shape"):
        sa.decode(q, kc, kc, max_splits=n, fused=True, out=torch.zeros(1, Hq, 1, d, device=dev, dtype=bf))
    with pytest.raises(ValueError, match="shape"):
        sa.decode(q, kc, kc, max_splits=n, fused=True, lse=torch.zeros(B, Hq - 1, device=dev, dtype=f32))
    with pytest.raises(ValueError, match="shape"):
        sa.decode(q, kc, kc, max_splits=n, out=torch.zeros(B, Hq, 2, d, device=dev, dtype=bf))
    T_q = 4
    qp = torch.zeros(B, Hq, T_q, d, device=dev, dtype=bf)
    pool = torch.zeros(6, Hkv, 64, d, device=dev, dtype=bf)
    table = torch.zeros(B, 3, device=dev, dtype=i32)
    lens = torch.full((B,), 100, device=dev, dtype=i32)
    with pytest.raises(ValueError, match="shape"):
        sa.decode_paged(qp, pool, pool, table, lens, 1, out=torch.zeros(B, Hq, 1, d, device=dev, dtype=bf))
    with pytest.raises(ValueError, match="shape"):
        sa.decode_paged(qp, pool, pool, table, lens, 1, lse=torch.zeros(B, Hq, 1, device=dev, dtype=f32))

"""ctypes binding of ``libattn.so`` -- argument marshalling only.

Every step of the attention computation runs in the library's HIP kernels; this
module checks tensor metadata, allocates outputs with torch (device memory),
passes raw pointers and torch's current HIP stream, and turns a non-zero
status into an exception.  There is no fallback: if the library is missing or
a call fails, an exception is raised.
"""

from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn.so")

ATTN_DTYPE_F32 = 0
ATTN_DTYPE_BF16 = 1
_DTYPE_CODE = {torch.float32: ATTN_DTYPE_F32, torch.bfloat16: ATTN_DTYPE_BF16}

STATUS = {0: "ATTN_OK", 1: "ATTN_ERR_NULL", 2: "ATTN_ERR_SHAPE", 3: "ATTN_ERR_UNSUPPORTED",
          4: "ATTN_ERR_ALIGN", 5: "ATTN_ERR_LAUNCH", 6: "ATTN_ERR_WORKSPACE"}
NOALLOC_MAX_PARTIALS = 65536   # ATTN_NOALLOC_MAX_PARTIALS

_P = ctypes.c_void_p
_I = ctypes.c_int32
_F = ctypes.c_float

SIGNATURES = {
    "attn_prefill": ([_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F, _P], ctypes.c_int),
    "attn_prefill_splitkv": ([_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _F, _P], ctypes.c_int),
    "attn_decode_splitkv": ([_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P, _P], ctypes.c_int),
    "attn_combine_lse": ([_P, _P, _P, _I, _I, _I, _I, _P, _P, _I, _P], ctypes.c_int),
    "attn_decode": ([_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P, _P, _P, _P, _P], ctypes.c_int),
    "attn_decode_noalloc": ([_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P, _P], ctypes.c_int),
    "attn_decode_paged": ([_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P, _P, _P, _P],
                          ctypes.c_int),
    "attn_status_string": ([ctypes.c_int], ctypes.c_char_p),
}

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = STATUS.get(status, f"status {status}")
        try:
            msg += ": " + lib().attn_status_string(status).decode()
        except Exception:  # pragma: no cover
            pass
        super().__init__(f"{where}: {msg}")


def lib():
    """Load ``libattn.so`` (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m streaming_attention_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need(t, name, ndim, dtype=None, device=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _check(status, where):
    if status != 0:
        raise AttnError(status, where)


def _check_prefill_args(q, k, v):
    _need(q, "q", 4)
    dt = q.dtype
    if dt not in _DTYPE_CODE:
        raise ValueError(f"unsupported dtype {dt}")
    _need(k, "k", 4, dt, q.device)
    _need(v, "v", 4, dt, q.device)
    B, Hq, Sq, d = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, Hkv, Skv, d) or tuple(v.shape) != (B, Hkv, Skv, d):
        raise ValueError(f"k/v shapes {tuple(k.shape)}, {tuple(v.shape)} do not match q {tuple(q.shape)}")
    return B, Hq, Hkv, Sq, Skv, d


# The bf16 prefill kernel runs 256 stacked query rows per workgroup and one
# workgroup per compute unit (its register budget); the MI355X has 256 CUs.
_PREFILL_ROWS_PER_WG = 256
_PREFILL_WG_TARGET = 256


def prefill_splits(B: int, Hq: int, Hkv: int, Sq: int, Skv: int, dtype=torch.bfloat16) -> int:
    """KV splits for a prefill: 1 when the query blocks alone fill the GPU
    (one workgroup per CU), else enough splits to reach that, keeping at least
    16 key tiles (1024 keys) per split.  A scheduling choice: any split count
    gives the same result up to rounding."""
    if dtype != torch.bfloat16:
        return 1
    blocks = -(-(Hq // Hkv) * Sq // _PREFILL_ROWS_PER_WG) * B * Hkv
    if blocks == 0 or blocks >= _PREFILL_WG_TARGET:
        return 1
    tiles = -(-Skv // 64)
    return int(max(1, min(-(-_PREFILL_WG_TARGET // blocks), tiles // 16, 256)))


def prefill_splitkv(q, k, v, num_splits: int, causal: bool = False, scale: float | None = None,
                    part_o=None, part_lse=None):
    """Split-KV prefill partials (``attn_prefill_splitkv``, bf16).

    Returns ``(part_o [B,Hq,Sq,num_splits,d] f32, part_lse [B,Hq,Sq,num_splits] f32)``;
    split ``s`` covers keys ``[64 s c, min(64 (s+1) c, Skv))`` with
    ``c = ceil(ceil(Skv/64) / num_splits)``.
    """
    B, Hq, Hkv, Sq, Skv, d = _check_prefill_args(q, k, v)
    if q.dtype != torch.bfloat16:
        raise ValueError("split-KV prefill takes bf16 inputs")
    n = int(num_splits)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if part_o is None:
        part_o = torch.empty((B, Hq, Sq, n, d), dtype=torch.float32, device=q.device)
    if part_lse is None:
        part_lse = torch.empty((B, Hq, Sq, n), dtype=torch.float32, device=q.device)
    _need(part_o, "part_o", 5, torch.float32, q.device)
    _need(part_lse, "part_lse", 4, torch.float32, q.device)
    if tuple(part_o.shape) != (B, Hq, Sq, n, d) or tuple(part_lse.shape) != (B, Hq, Sq, n):
        raise ValueError("partial buffers must be [B,Hq,Sq,num_splits,d] and [B,Hq,Sq,num_splits]")
    st = lib().attn_prefill_splitkv(_ptr(q), _ptr(k), _ptr(v), _ptr(part_o), _ptr(part_lse), B, Hq, Hkv, Sq,
                                    Skv, d, n, ATTN_DTYPE_BF16, 1 if causal else 0, float(scale), _stream(q))
    _check(st, "attn_prefill_splitkv")
    return part_o, part_lse


def prefill(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None,
            return_lse: bool = True, num_splits: int | None = None):
    """Fused streaming attention forward.

    ``q [B,Hq,Sq,d]``, ``k, v [B,Hkv,Skv,d]``, bf16 or fp32, contiguous, on one
    GPU.  Causal alignment is bottom-right (the queries are the last Sq
    positions).  ``num_splits`` None picks ``prefill_splits(...)``: 1 runs
    ``attn_prefill``; more runs ``attn_prefill_splitkv`` and merges the
    partials with ``attn_combine_lse`` (bf16 only).  Returns ``(o, lse)`` or ``o``.
    """
    B, Hq, Hkv, Sq, Skv, d = _check_prefill_args(q, k, v)
    dt = q.dtype
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    else:
        _need(out, "out", 4, dt, q.device)
        if out.shape != q.shape:
            raise ValueError("out must have the shape of q")
    if return_lse and lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", 3, torch.float32, q.device)
        if tuple(lse.shape) != (B, Hq, Sq):
            raise ValueError("lse must be [B,Hq,Sq]")
    n = prefill_splits(B, Hq, Hkv, Sq, Skv, dt) if num_splits is None else int(num_splits)
    if n == 1:
        st = lib().attn_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, Sq, Skv, d,
                                _DTYPE_CODE[dt], 1 if causal else 0, float(scale), _stream(q))
        _check(st, "attn_prefill")
    else:
        po, pl = prefill_splitkv(q, k, v, n, causal, scale)
        st = lib().attn_combine_lse(_ptr(po), _ptr(pl), None, B * Hq * Sq, 1, n, d, _ptr(out), _ptr(lse),
                                    _DTYPE_CODE[dt], _stream(q))
        _check(st, "attn_combine_lse")
    return (out, lse) if return_lse else out


def decode_splitkv(q, k_cache, v_cache, kv_len=None, num_splits=None, max_splits: int = 64,
                   scale: float | None = None, part_o=None, part_lse=None):
    """Split-KV decode partials (``attn_decode_splitkv``).

    ``q [B,Hq,1,d]`` bf16, caches ``[B,Hkv,S_cap,d]`` bf16, ``kv_len`` and
    ``num_splits`` int32 GPU tensors ``[B]`` or None.  Returns
    ``(part_o [B,Hq,max_splits,d] f32, part_lse [B,Hq,max_splits] f32)``.
    """
    _need(q, "q", 4, torch.bfloat16)
    _need(k_cache, "k_cache", 4, torch.bfloat16, q.device)
    _need(v_cache, "v_cache", 4, torch.bfloat16, q.device)
    B, Hq, one, d = q.shape
    if one != 1:
        raise ValueError("decode takes one query token per sequence: q must be [B,Hq,1,d]")
    Hkv, S_cap = k_cache.shape[1], k_cache.shape[2]
    if tuple(k_cache.shape) != (B, Hkv, S_cap, d) or v_cache.shape != k_cache.shape:
        raise ValueError("cache shapes do not match q")
    for name, t in (("kv_len", kv_len), ("num_splits", num_splits)):
        if t is not None:
            _need(t, name, 1, torch.int32, q.device)
            if t.shape[0] != B:
                raise ValueError(f"{name} must have B entries")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if part_o is None:
        part_o = torch.empty((B, Hq, max_splits, d), dtype=torch.float32, device=q.device)
    if part_lse is None:
        part_lse = torch.empty((B, Hq, max_splits), dtype=torch.float32, device=q.device)
    _need(part_o, "part_o", 4, torch.float32, q.device)
    _need(part_lse, "part_lse", 3, torch.float32, q.device)
    if tuple(part_o.shape) != (B, Hq, max_splits, d) or tuple(part_lse.shape) != (B, Hq, max_splits):
        raise ValueError("partial buffers must be [B,Hq,max_splits,d] and [B,Hq,max_splits]")
    st = lib().attn_decode_splitkv(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(kv_len), _ptr(num_splits),
                                   B, Hq, Hkv, S_cap, d, int(max_splits), ATTN_DTYPE_BF16, float(scale),
                                   _ptr(part_o), _ptr(part_lse), _stream(q))
    _check(st, "attn_decode_splitkv")
    return part_o, part_lse


def combine_lse(part_o, part_lse, num_splits=None, out_dtype=torch.bfloat16, out=None, lse=None):
    """Log-sum-exp merge of split partials (``attn_combine_lse``).

    Returns ``(o [B,Hq,1,d] out_dtype, lse [B,Hq] f32)``.
    """
    _need(part_o, "part_o", 4, torch.float32)
    B, Hq, max_splits, d = part_o.shape
    _need(part_lse, "part_lse", 3, torch.float32, part_o.device)
    if tuple(part_lse.shape) != (B, Hq, max_splits):
        raise ValueError("part_lse must be [B,Hq,max_splits]")
    if num_splits is not None:
        _need(num_splits, "num_splits", 1, torch.int32, part_o.device, (B,))
    if out_dtype not in _DTYPE_CODE:
        raise ValueError(f"unsupported out_dtype {out_dtype}")
    if out is None:
        out = torch.empty((B, Hq, 1, d), dtype=out_dtype, device=part_o.device)
    _need(out, "out", 4, out_dtype, part_o.device, (B, Hq, 1, d))
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=part_o.device)
    _need(lse, "lse", 2, torch.float32, part_o.device, (B, Hq))
    st = lib().attn_combine_lse(_ptr(part_o), _ptr(part_lse), _ptr(num_splits), B, Hq, max_splits, d,
                                _ptr(out), _ptr(lse), _DTYPE_CODE[out_dtype], _stream(part_o))
    _check(st, "attn_combine_lse")
    return out, lse


_COUNTERS = {}


def _counters_for(device, n):
    """A zeroed int32 counter workspace of at least n entries, cached per device.

    attn_decode leaves it zero again after every launch, so it can be reused by
    launches that are ordered on one stream.  Callers that launch concurrently
    on several streams pass their own buffers.
    """
    t = _COUNTERS.get(device)
    if t is None or t.numel() < n:
        t = torch.zeros(max(n, 256), dtype=torch.int32, device=device)
        _COUNTERS[device] = t
    return t


def decode(q, k_cache, v_cache, kv_len=None, num_splits=None, max_splits: int = 64,
           scale: float | None = None, part_o=None, part_lse=None, out=None, lse=None,
           counters=None, fused: bool = False):
    """Split-KV decode followed by the log-sum-exp merge: ``(o, lse)``.

    ``fused=False`` (default) runs ``attn_decode_splitkv`` then
    ``attn_combine_lse`` -- the faster path for large decodes.  ``fused=True``
    runs both in one launch (``attn_decode``; ``counters`` is an int32
    workspace of ``B * Hkv`` zeros, a cached one when None).
    """
    if not fused:
        po, pl = decode_splitkv(q, k_cache, v_cache, kv_len, num_splits, max_splits, scale, part_o, part_lse)
        return combine_lse(po, pl, num_splits, q.dtype, out, lse)
    _need(q, "q", 4, torch.bfloat16)
    _need(k_cache, "k_cache", 4, torch.bfloat16, q.device)
    _need(v_cache, "v_cache", 4, torch.bfloat16, q.device)
    B, Hq, one, d = q.shape
    if one != 1:
        raise ValueError("decode takes one query token per sequence: q must be [B,Hq,1,d]")
    Hkv, S_cap = k_cache.shape[1], k_cache.shape[2]
    if tuple(k_cache.shape) != (B, Hkv, S_cap, d) or v_cache.shape != k_cache.shape:
        raise ValueError("cache shapes do not match q")
    for name, t in (("kv_len", kv_len), ("num_splits", num_splits)):
        if t is not None:
            _need(t, name, 1, torch.int32, q.device)
            if t.shape[0] != B:
                raise ValueError(f"{name} must have B entries")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if part_o is None:
        part_o = torch.empty((B, Hq, max_splits, d), dtype=torch.float32, device=q.device)
    if part_lse is None:
        part_lse = torch.empty((B, Hq, max_splits), dtype=torch.float32, device=q.device)
    _need(part_o, "part_o", 4, torch.float32, q.device)
    _need(part_lse, "part_lse", 3, torch.float32, q.device)
    if tuple(part_o.shape) != (B, Hq, max_splits, d) or tuple(part_lse.shape) != (B, Hq, max_splits):
        raise ValueError("partial buffers must be [B,Hq,max_splits,d] and [B,Hq,max_splits]")
    if counters is None:
        counters = _counters_for(q.device, B * Hkv)
    _need(counters, "counters", 1, torch.int32, q.device)
    if counters.numel() < B * Hkv:
        raise ValueError("counters must hold B * Hkv entries")
    if out is None:
        out = torch.empty((B, Hq, 1, d), dtype=torch.bfloat16, device=q.device)
    _need(out, "out", 4, torch.bfloat16, q.device, (B, Hq, 1, d))
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _need(lse, "lse", 2, torch.float32, q.device, (B, Hq))
    st = lib().attn_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(kv_len), _ptr(num_splits),
                           B, Hq, Hkv, S_cap, d, int(max_splits), ATTN_DTYPE_BF16, float(scale),
                           _ptr(part_o), _ptr(part_lse), _ptr(counters), _ptr(out), _ptr(lse), _stream(q))
    _check(st, "attn_decode")
    return out, lse


def decode_noalloc(q, k_cache, v_cache, kv_len=None, num_splits=None, max_splits: int = 64,
                   scale: float | None = None, out=None, lse=None):
    """Split-KV decode + merge with the partials in the library's fixed
    workspace (``attn_decode_noalloc``): the launch itself allocates nothing.
    Pass ``out [B,Hq,1,d]`` bf16 and ``lse [B,Hq]`` f32 to allocate nothing
    here either.  Requires ``B * Hq * max_splits <= 65536``.  Calls that
    overlap in time on one GPU share the workspace and race."""
    _need(q, "q", 4, torch.bfloat16)
    _need(k_cache, "k_cache", 4, torch.bfloat16, q.device)
    _need(v_cache, "v_cache", 4, torch.bfloat16, q.device)
    B, Hq, one, d = q.shape
    if one != 1:
        raise ValueError("decode takes one query token per sequence: q must be [B,Hq,1,d]")
    Hkv, S_cap = k_cache.shape[1], k_cache.shape[2]
    if tuple(k_cache.shape) != (B, Hkv, S_cap, d) or v_cache.shape != k_cache.shape:
        raise ValueError("cache shapes do not match q")
    for name, t in (("kv_len", kv_len), ("num_splits", num_splits)):
        if t is not None:
            _need(t, name, 1, torch.int32, q.device, (B,))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, Hq, 1, d), dtype=torch.bfloat16, device=q.device)
    _need(out, "out", 4, torch.bfloat16, q.device, (B, Hq, 1, d))
    if lse is not None:
        _need(lse, "lse", 2, torch.float32, q.device, (B, Hq))
    st = lib().attn_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(kv_len), _ptr(num_splits),
                                   B, Hq, Hkv, S_cap, d, int(max_splits), ATTN_DTYPE_BF16, float(scale),
                                   _ptr(out), _ptr(lse), _stream(q))
    _check(st, "attn_decode_noalloc")
    return out, lse


PAGE = 64   # positions per KV-cache page (the kernels' key tile)


def paged_splits(B: int, Hq: int, Hkv: int, T_q: int, max_pages: int) -> int:
    """Default split count of ``decode_paged``, the same for every sequence.

    Query blocks of at most 32 stacked rows (G * T_q <= 32) run the streaming
    paged decode kernel, two workgroups per compute unit: aim at about 768
    (sequence, KV head, split) workgroups, three per compute unit, so that
    the short sequences' workgroups fill in around the long ones.  Larger
    query blocks run the prefill kernel's paged mode: about 1024 (query
    block, split) workgroups.  Either way at least 8 pages of the longest
    possible sequence go to a split.  Measured on 16 sequences of 1K-32K keys
    (8 heads x 4 tokens): 6 splits beat 4, 8, 10, 12 and 16, and beat splits
    sized per sequence.  Any split count gives the same result up to rounding."""
    rows = (Hq // Hkv) * T_q
    if rows <= 32:
        blocks, target = B * Hkv, 768
    else:
        blocks, target = -(-rows // 128) * B * Hkv, 1024
    if blocks == 0:
        return 1
    return int(max(1, min(-(-target // blocks), max_pages // 8, 256)))


def decode_paged(q, k_pages, v_pages, block_table, kv_len, num_splits: int | None = None,
                 scale: float | None = None, out=None, lse=None, keys_per_split: int | None = None):
    """Multi-token decode over a paged KV cache (``attn_decode_paged``).

    ``q [B,Hq,T_q,d]`` bf16; ``k_pages, v_pages [num_pages,Hkv,64,d]`` bf16;
    ``block_table [B,max_pages]`` and ``kv_len [B]`` int32 GPU tensors.  Each
    sequence's T_q tokens are its last T_q positions.  ``keys_per_split``
    given: sequence b takes ``ceil(kv_len[b] / keys_per_split)`` splits
    (computed on the GPU); otherwise every sequence takes ``num_splits``
    (None: ``paged_splits``).  More than one split is merged by
    ``attn_combine_lse``.  Returns ``(o [B,Hq,T_q,d] bf16, lse [B,Hq,T_q] f32)``.
    """
    _need(q, "q", 4, torch.bfloat16)
    _need(k_pages, "k_pages", 4, torch.bfloat16, q.device)
    _need(v_pages, "v_pages", 4, torch.bfloat16, q.device)
    _need(block_table, "block_table", 2, torch.int32, q.device)
    _need(kv_len, "kv_len", 1, torch.int32, q.device)
    B, Hq, T_q, d = q.shape
    num_pages, Hkv, page, dk = k_pages.shape
    if page != PAGE or dk != d or v_pages.shape != k_pages.shape:
        raise ValueError(f"page pools must be [num_pages,Hkv,{PAGE},d] and alike")
    if block_table.shape[0] != B or kv_len.shape[0] != B:
        raise ValueError("block_table and kv_len need B rows")
    max_pages = block_table.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    seq = None
    if keys_per_split is not None:
        kps = int(keys_per_split)
        n = int(max(1, min(256, -(-max_pages * PAGE // kps))))
        if n > 1:
            seq = ((kv_len + (kps - 1)) // kps).clamp(1, n).to(torch.int32)
    elif num_splits is None:
        n = paged_splits(B, Hq, Hkv, T_q, max_pages)
    else:
        n = int(num_splits)
    if out is None:
        out = torch.empty((B, Hq, T_q, d), dtype=torch.bfloat16, device=q.device)
    _need(out, "out", 4, torch.bfloat16, q.device, (B, Hq, T_q, d))
    if lse is None:
        lse = torch.empty((B, Hq, T_q), dtype=torch.float32, device=q.device)
    _need(lse, "lse", 3, torch.float32, q.device, (B, Hq, T_q))
    po = pl = None
    if n > 1:
        po = torch.empty((B, Hq, T_q, n, d), dtype=torch.float32, device=q.device)
        pl = torch.empty((B, Hq, T_q, n), dtype=torch.float32, device=q.device)
    st = lib().attn_decode_paged(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), _ptr(kv_len), _ptr(seq),
                                 B, Hq, Hkv, T_q, num_pages, max_pages, d, n, ATTN_DTYPE_BF16, float(scale),
                                 _ptr(po), _ptr(pl), _ptr(out), _ptr(lse), _stream(q))
    _check(st, "attn_decode_paged")
    if n > 1:
        st = lib().attn_combine_lse(_ptr(po), _ptr(pl), _ptr(seq), B, Hq * T_q, n, d, _ptr(out), _ptr(lse),
                                    ATTN_DTYPE_BF16, _stream(q))
        _check(st, "attn_combine_lse")
    return out, lse


def splits_for_lengths(lens, keys_per_split: int = 2048, max_splits: int = 64):
    """Split count per sequence: ``min(max_splits, max(1, ceil(len / keys_per_split)))``.

    A tuning choice (the pages leave the one-shot vs tiled crossover open); any
    split count gives the same result up to rounding.
    """
    lens = torch.as_tensor(lens, dtype=torch.int64)
    n = (lens + keys_per_split - 1) // keys_per_split
    return n.clamp(1, max_splits).to(torch.int32)

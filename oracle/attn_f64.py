"""Plain float64 attention: the definition written out, plus the pages' tile
recurrence and log-sum-exp merge, for checking the GPU library.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Nothing here is tuned,
blocked or fused beyond what the cited passage states.

Conventions shared with the tests (they are the method's statement of the
problem, not GPU implementation details):
  * Q is ``[B, Hq, Sq, d]``; K and V are ``[B, Hkv, Skv, d]``; ``G = Hq // Hkv``
    and query head ``h`` reads KV head ``h // G`` (the G query heads of one KV
    head are consecutive -- ADR-0060, section 0 "CUBE Group" and section 5.2,
    where the group's query rows are stacked into the GEMM M dimension).
  * The scale multiplies ``Q K^T`` before the mask and the softmax (ADR-0060
    section 3: the score GEMM is multiplied by ``softmax_scale``; section 0.5.3
    gives ``1/sqrt(d)`` as its value).
  * Causal alignment is bottom-right: query row ``t`` sits at global position
    ``q_start + t`` with ``q_start = Skv - Sq`` and sees key ``j`` iff
    ``j <= q_start + t`` (ADR-0060 section 0.5.3: ``q_block_meta {q_start,
    T_q}`` carries the query block's global position; section 5.4 classifies
    tiles by ``[qs, qe)`` against ``[ks, ke)``).  The diagonal is visible.
  * ``kv_len[b]`` hides keys ``j >= kv_len[b]`` (ADR-0060 section 5.2: only the
    last ragged tile is masked).
  * Natural exponential and logarithm throughout; ``LSE = m + ln(l)``.
  * A row with no visible key yields ``O = 0`` and ``LSE = -inf``.
"""

from __future__ import annotations


import numpy as np


def _f64(x) -> np.ndarray:
    """Exact widening to float64 (bf16 and fp32 values are representable)."""
    return np.asarray(x, dtype=np.float64)


def visible_keys(Sq: int, Skv: int, causal: bool, kv_len: int | None = None,
                 rows=None) -> np.ndarray:
    """Boolean ``[n_rows, Skv]`` visibility of key ``j`` to query row ``t``.

    Causal pattern: "AI Compiler pipeline stages", Pattern Matching (a causal
    mask between the score product and the softmax); alignment per ADR-0060
    section 0.5.3 / 5.4 (bottom-right, diagonal included).  ``kv_len`` per
    ADR-0060 section 5.2 (ragged last tile).
    """
    t = np.arange(Sq) if rows is None else np.asarray(rows, dtype=np.int64)
    j = np.arange(Skv)
    vis = np.ones((t.shape[0], Skv), dtype=bool)
    if causal:
        q_start = Skv - Sq
        vis &= j[None, :] <= (q_start + t)[:, None]
    if kv_len is not None:
        vis &= j[None, :] < int(kv_len)
    return vis


def _head(qh: np.ndarray, kh: np.ndarray, vh: np.ndarray, scale: float,
          vis: np.ndarray):
    """Two-pass stable softmax attention for one head, score matrix materialised.

    The stable form ``exp(x - max x) / sum exp(x - max x)`` is the canonical
    softmax of "AI Compiler pipeline stages" (IR Normalization).  Returns
    ``(O [n, d], LSE [n])`` in float64.
    """
    S = scale * (qh @ kh.T)                          # [n, Skv]
    S = np.where(vis, S, -np.inf)
    m = S.max(axis=1, initial=-np.inf)               # -inf on empty rows (and for Skv = 0)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    E = np.where(vis, np.exp(S - m_safe[:, None]), 0.0)
    l = E.sum(axis=1)
    has = l > 0
    P = np.where(has[:, None], E / np.where(has, l, 1.0)[:, None], 0.0)
    O = P @ vh
    with np.errstate(divide="ignore"):
        lse = np.where(has, m_safe + np.log(np.where(has, l, 1.0)), -np.inf)
    return O, lse


def attention(q, k, v, scale: float, causal: bool = False, kv_len=None):
    """Scaled-dot-product attention by its definition, float64.

    ``O = softmax_rows(scale * Q K^T masked) V`` -- the attention region the
    pages start from ("AttentionRegion Transformation", sections 3-4: score
    matmul, optional mask, softmax, value matmul).

    ``q [B,Hq,Sq,d]``, ``k, v [B,Hkv,Skv,d]``, ``kv_len`` None or length-B.
    Returns ``O [B,Hq,Sq,d]`` and ``LSE [B,Hq,Sq]`` (float64).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Sq, d = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    assert Hq % Hkv == 0
    G = Hq // Hkv
    O = np.zeros((B, Hq, Sq, v.shape[3]))
    L = np.zeros((B, Hq, Sq))
    for b in range(B):
        vis = visible_keys(Sq, Skv, causal,
                           None if kv_len is None else int(kv_len[b]))
        for h in range(Hq):
            kv = h // G
            O[b, h], L[b, h] = _head(q[b, h], k[b, kv], v[b, kv], scale, vis)
    return O, L


def attention_rows(q, k, v, scale: float, causal: bool, b: int, h: int, rows,
                   kv_len=None):
    """The same definition evaluated for selected query rows of head ``(b, h)``.

    Used at full problem sizes, where the whole score matrix would not fit the
    time budget of a test.  Only the requested rows' scores are formed.
    """
    Hq, Sq = q.shape[1], q.shape[2]
    Hkv, Skv = k.shape[1], k.shape[2]
    kv = h // (Hq // Hkv)
    rows = np.asarray(rows, dtype=np.int64)
    vis = visible_keys(Sq, Skv, causal, kv_len, rows=rows)
    return _head(_f64(q[b, h][rows]), _f64(k[b, kv]), _f64(v[b, kv]), scale, vis)


def attention_online(q, k, v, scale: float, causal: bool = False, tile: int = 64,
                     kv_len=None):
    """The pages' streaming algorithm, float64: KV tiles visited in order with a
    running max ``m``, running sum ``l`` and rescaled output accumulator ``O``.

    Follows ADR-0060 section 3 (per-tile sequence: scores, boundary mask, tile
    max, new max, ``P = exp(S - m_new)``, ``corr = exp(m - m_new)``,
    ``l = l*corr + rowsum(P)``, ``O = O*corr + P V``, ``m = m_new``; initial
    state ``(-inf, 0, 0)``; ``O / l`` once at the end) and its section 5.4 tile
    classes (tiles wholly in the future are skipped, tiles wholly in the past
    take no mask, straddling tiles take the triangular mask).  The recurrence
    for ``m`` and ``l`` is also the one in "AttentionRegion Transformation"
    section 6.  A row that has seen no key keeps ``m = -inf``; its correction
    factor ``exp(-inf - (-inf))`` is taken as 0.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Sq, d = q.shape
    Hkv, Skv, dv = k.shape[1], k.shape[2], v.shape[3]
    G = Hq // Hkv
    q_start = Skv - Sq
    O_all = np.zeros((B, Hq, Sq, dv))
    L_all = np.zeros((B, Hq, Sq))
    for b in range(B):
        n_valid = Skv if kv_len is None else int(kv_len[b])
        for h in range(Hq):
            kv = h // G
            qh = q[b, h]
            m = np.full(Sq, -np.inf)
            l = np.zeros(Sq)
            O = np.zeros((Sq, dv))
            qs, qe = q_start, q_start + Sq          # global positions of the block
            n_tiles = -(-n_valid // tile)
            for jt in range(n_tiles):
                ks, ke = jt * tile, min((jt + 1) * tile, n_valid)
                if causal and ks >= qe:
                    continue                         # whole tile in the future
                S = scale * (qh @ k[b, kv, ks:ke].T)
                if causal and ke - 1 > qs:           # tile straddles the diagonal
                    pos = q_start + np.arange(Sq)
                    S = np.where(np.arange(ks, ke)[None, :] <= pos[:, None], S, -np.inf)
                m_j = S.max(axis=1)
                m_new = np.maximum(m, m_j)
                base = np.where(np.isfinite(m_new), m_new, 0.0)
                P = np.exp(S - base[:, None])        # exp(-inf) = 0 for masked keys
                corr = np.where(np.isfinite(m), np.exp(m - base), 0.0)
                l = l * corr + P.sum(axis=1)
                O = O * corr[:, None] + P @ v[b, kv, ks:ke]
                m = m_new
            has = l > 0
            O_all[b, h] = np.where(has[:, None], O / np.where(has, l, 1.0)[:, None], 0.0)
            with np.errstate(divide="ignore"):
                L_all[b, h] = np.where(has, m + np.log(np.where(has, l, 1.0)), -np.inf)
    return O_all, L_all


def partial_attention(q, k, v, scale: float, key_lo: int, key_hi: int):
    """One split's result over keys ``[key_lo, key_hi)`` for decode queries.

    ADR-0060 section 4: after its sweep each split holds an unnormalised
    ``(m_i, l_i, O_i)`` over its own key range.  This returns the equivalent
    normalised pair ``(lse_i = m_i + ln l_i, O_i / l_i)``; an empty range gives
    ``(-inf, 0)``.

    ``q [Hq, d]`` (one sequence, one query token), ``k, v [Hkv, S, d]``.
    Returns ``lse [Hq]`` and ``O [Hq, d]`` (float64).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    Hq, Hkv = q.shape[0], k.shape[0]
    G = Hq // Hkv
    O = np.zeros((Hq, v.shape[2]))
    L = np.full(Hq, -np.inf)
    if key_hi <= key_lo:
        return L, O
    vis = np.ones((1, key_hi - key_lo), dtype=bool)
    for h in range(Hq):
        kv = h // G
        o, lse = _head(q[h][None, :], k[kv, key_lo:key_hi], v[kv, key_lo:key_hi],
                       scale, vis)
        O[h], L[h] = o[0], lse[0]
    return L, O


def attention_key_range(q, k, v, scale: float, causal: bool, key_lo: int, key_hi: int):
    """One split's result for every query row of a prefill: the definition with
    only keys ``[key_lo, key_hi)`` (and, when causal, the usual diagonal mask)
    visible.

    On one device the pages' ring prefill ("ADR-0060", section 5.5: every step
    folds one K/V block into the running state of each query block) and the
    split partials of section 4 both reduce to this: each block of keys yields
    a normalised pair ``(lse_i, O_i)`` for every query row, merged afterwards
    by ``merge_partials``.  A row that sees no key of the range gives
    ``(-inf, 0)``.

    ``q [B,Hq,Sq,d]``, ``k, v [B,Hkv,Skv,d]``.  Returns ``O [B,Hq,Sq,d]`` and
    ``LSE [B,Hq,Sq]`` (float64).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Sq, d = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    vis = visible_keys(Sq, Skv, causal)
    j = np.arange(Skv)
    vis &= ((j >= key_lo) & (j < key_hi))[None, :]
    O = np.zeros((B, Hq, Sq, v.shape[3]))
    L = np.zeros((B, Hq, Sq))
    for b in range(B):
        for h in range(Hq):
            O[b, h], L[b, h] = _head(q[b, h], k[b, h // G], v[b, h // G], scale, vis)
    return O, L


def merge_partials(lse_parts, o_parts):
    """Combine partial results with the pages' log-sum-exp merge, float64.

    ADR-0060 section 4: ``m = max(m_a, m_b)``, ``s_a = exp(m_a - m)``,
    ``s_b = exp(m_b - m)``, result ``(m, l_a s_a + l_b s_b, O_a s_a + O_b s_b)``;
    the output is normalised once at the end (``O / l``).  A normalised partial
    ``(lse, O)`` enters as the triplet ``(m = lse, l = 1, O)``; an empty one as
    ``(-inf, 0, 0)``.  ``lse_parts [n, ...]``, ``o_parts [n, ..., d]`` are folded
    left to right along axis 0.  Returns ``(lse, O)``.
    """
    lse_parts = _f64(lse_parts)
    o_parts = _f64(o_parts)
    m = np.full(lse_parts.shape[1:], -np.inf)
    l = np.zeros(lse_parts.shape[1:])
    O = np.zeros(o_parts.shape[1:])
    for i in range(lse_parts.shape[0]):
        m_b = lse_parts[i]
        l_b = np.where(np.isfinite(m_b), 1.0, 0.0)
        O_b = np.where(np.isfinite(m_b)[..., None], o_parts[i], 0.0)
        m_new = np.maximum(m, m_b)
        base = np.where(np.isfinite(m_new), m_new, 0.0)
        s_a = np.where(np.isfinite(m), np.exp(m - base), 0.0)
        s_b = np.where(np.isfinite(m_b), np.exp(m_b - base), 0.0)
        m = m_new
        l = l * s_a + l_b * s_b
        O = O * s_a[..., None] + O_b * s_b[..., None]
    has = l > 0
    O_out = np.where(has[..., None], O / np.where(has, l, 1.0)[..., None], 0.0)
    with np.errstate(divide="ignore"):
        lse = np.where(has, m + np.log(np.where(has, l, 1.0)), -np.inf)
    return lse, O_out


def decode_attention(q, k_cache, v_cache, kv_len, scale: float):
    """Single-token decode: each sequence's query attends to all its valid keys.

    ADR-0060 section 5.2: decode has ``T_q = 1`` and attends to all past KV
    (the new token's K/V row was appended upstream before the launch, section
    0.5.1), so only the ragged last tile is masked.  ``q [B, Hq, d]`` or
    ``[B, Hq, 1, d]``; caches ``[B, Hkv, S_cap, d]``.  Returns ``O [B, Hq, d]``
    and ``LSE [B, Hq]``.
    """
    q = _f64(q)
    if q.ndim == 3:
        q = q[:, :, None, :]
    O, L = attention(q, k_cache, v_cache, scale, causal=False, kv_len=kv_len)
    return O[:, :, 0, :], L[:, :, 0]


def paged_attention(q, k_pages, v_pages, block_table, kv_len, scale: float):
    """Multi-token decode over a paged KV cache: every sequence's ``T_q`` query
    tokens are the last ``T_q`` positions of its ``kv_len[b]`` valid keys and
    attend causally (bottom-right) to them.

    "ADR-0060" section 0.5.3: the query block carries its global start and
    length (``q_block_meta {q_start, T_q}``, here ``q_start = kv_len[b] - T_q``),
    and the kernel derives its valid length from a counter (section 2.2,
    ``my_len``; here ``kv_len[b]``).  Section 2.1 lets the keys of a sequence sit
    in a non-contiguous placement that plain arithmetic maps back to global
    positions; here that map is a block table: logical page ``p`` of sequence
    ``b`` (keys ``p*page .. p*page + page - 1``) is physical page
    ``block_table[b, p]`` of the pool.

    ``q [B, Hq, T_q, d]``; ``k_pages, v_pages [num_pages, Hkv, page, d]``;
    ``block_table [B, max_pages]`` (entries past a sequence's last page are
    ignored); ``kv_len [B]``.  The sequence's keys are gathered page by page
    into a contiguous ``[Hkv, kv_len[b], d]`` cache and the definition
    (``attention``, causal) is applied to it.  Returns ``O [B, Hq, T_q, d]`` and
    ``LSE [B, Hq, T_q]`` (float64).
    """
    q, k_pages, v_pages = _f64(q), _f64(k_pages), _f64(v_pages)
    block_table = np.asarray(block_table, dtype=np.int64)
    B, Hq, T_q, d = q.shape
    page = k_pages.shape[2]
    O = np.zeros((B, Hq, T_q, v_pages.shape[3]))
    L = np.zeros((B, Hq, T_q))
    Hkv, dk, dv = k_pages.shape[1], k_pages.shape[3], v_pages.shape[3]
    for b in range(B):
        n = int(kv_len[b])
        ids = block_table[b, :-(-n // page)]
        kb = np.concatenate([np.zeros((Hkv, 0, dk))] + [k_pages[i] for i in ids], axis=1)[:, :n]
        vb = np.concatenate([np.zeros((Hkv, 0, dv))] + [v_pages[i] for i in ids], axis=1)[:, :n]
        O[b], L[b] = attention(q[b:b + 1], kb[None], vb[None], scale, True)
    return O, L


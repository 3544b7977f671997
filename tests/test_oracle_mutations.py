"""Plant plausible mistakes in the oracle (on the CPU) and show that the pins
catch each one.  A pin set that still passed with a planted mistake would not
be pinning that part of the oracle."""

import numpy as np
import pytest

import oracle
import oracle.attn_f64 as oa
from oracle_pins import ALL_CHECKS


def _any_check_fails():
    failed = []
    for check in ALL_CHECKS:
        try:
            check()
        except AssertionError as e:  # noqa: PERF203
            failed.append((check.__name__, str(e)[:80]))
    return failed


def _top_left_visible(Sq, Skv, causal, kv_len=None, rows=None):
    t = np.arange(Sq) if rows is None else np.asarray(rows)
    j = np.arange(Skv)
    vis = np.ones((t.shape[0], Skv), dtype=bool)
    if causal:
        vis &= j[None, :] <= t[:, None]          # mistake: no q_start offset
    if kv_len is not None:
        vis &= j[None, :] < int(kv_len)
    return vis


def _strict_diagonal(Sq, Skv, causal, kv_len=None, rows=None):
    t = np.arange(Sq) if rows is None else np.asarray(rows)
    j = np.arange(Skv)
    vis = np.ones((t.shape[0], Skv), dtype=bool)
    if causal:
        vis &= j[None, :] < (Skv - Sq + t)[:, None]   # mistake: diagonal hidden
    if kv_len is not None:
        vis &= j[None, :] < int(kv_len)
    return vis


def _head_no_max_shift(qh, kh, vh, scale, vis):
    S = scale * (qh @ kh.T)
    E = np.where(vis, np.exp(np.where(vis, S, 0.0)), 0.0)
    l = E.sum(axis=1)
    O = (E / l[:, None]) @ vh
    return O, np.log(l) + 1e-6                   # mistake: LSE off by a hair


def _head_scale_after_softmax(qh, kh, vh, scale, vis):
    S = qh @ kh.T                               # mistake: scale dropped
    S = np.where(vis, S, -np.inf)
    m = S.max(axis=1)
    E = np.where(vis, np.exp(S - m[:, None]), 0.0)
    l = E.sum(axis=1)
    return (E / l[:, None]) @ vh, m + np.log(l)


def _head_transposed_v(qh, kh, vh, scale, vis):
    O, L = ORIG_HEAD(qh, kh, vh, scale, vis)
    if vh.shape[0] == vh.shape[1] and vh.shape[0] > 1:
        O = ORIG_HEAD(qh, kh, vh.T.copy(), scale, vis)[0]   # mistake: V transposed
    else:
        O = O[:, ::-1].copy()                    # mistake: value columns reversed
    return O, L


ORIG_HEAD = oa._head


def _attention_wrong_head_map(q, k, v, scale, causal=False, kv_len=None):
    q, k, v = oa._f64(q), oa._f64(k), oa._f64(v)
    B, Hq, Sq, _ = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    O = np.zeros((B, Hq, Sq, v.shape[3]))
    L = np.zeros((B, Hq, Sq))
    for b in range(B):
        vis = oa.visible_keys(Sq, Skv, causal, None if kv_len is None else int(kv_len[b]))
        for h in range(Hq):
            O[b, h], L[b, h] = oa._head(q[b, h], k[b, h % Hkv], v[b, h % Hkv], scale, vis)
    return O, L


def _online_no_rescale(q, k, v, scale, causal=False, tile=64, kv_len=None):
    """Recurrence with the O rescale left out (the omission one page makes)."""
    q, k, v = oa._f64(q), oa._f64(k), oa._f64(v)
    B, Hq, Sq, d = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    O_all = np.zeros((B, Hq, Sq, v.shape[3]))
    L_all = np.zeros((B, Hq, Sq))
    q_start = Skv - Sq
    for b in range(B):
        n_valid = Skv if kv_len is None else int(kv_len[b])
        for h in range(Hq):
            m = np.full(Sq, -np.inf)
            l = np.zeros(Sq)
            O = np.zeros((Sq, v.shape[3]))
            for ks in range(0, n_valid, tile):
                ke = min(ks + tile, n_valid)
                S = scale * (q[b, h] @ k[b, h // G, ks:ke].T)
                if causal:
                    pos = q_start + np.arange(Sq)
                    S = np.where(np.arange(ks, ke)[None, :] <= pos[:, None], S, -np.inf)
                m_new = np.maximum(m, S.max(axis=1))
                base = np.where(np.isfinite(m_new), m_new, 0.0)
                P = np.exp(S - base[:, None])
                corr = np.where(np.isfinite(m), np.exp(m - base), 0.0)
                l = l * corr + P.sum(axis=1)
                O = O + P @ v[b, h // G, ks:ke]      # mistake: no O * corr
                m = m_new
            O_all[b, h] = O / np.maximum(l, 1e-300)[:, None]
            L_all[b, h] = m + np.log(np.maximum(l, 1e-300))
    return O_all, L_all


def _merge_wrong_sign(lse_parts, o_parts):
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    return ORIG_MERGE(-lse_parts, o_parts)       # mistake: weights e^{-lse}


ORIG_MERGE = oa.merge_partials


def _partial_off_by_one(q, k, v, scale, key_lo, key_hi):
    return ORIG_PARTIAL(q, k, v, scale, key_lo, max(key_lo, key_hi - 1))


ORIG_PARTIAL = oa.partial_attention


def _key_range_half_open_wrong(q, k, v, scale, causal, key_lo, key_hi):
    return ORIG_KEY_RANGE(q, k, v, scale, causal, key_lo, key_hi + 1)   # mistake: range includes key_hi


def _key_range_no_causal(q, k, v, scale, causal, key_lo, key_hi):
    return ORIG_KEY_RANGE(q, k, v, scale, False, key_lo, key_hi)        # mistake: mask dropped


ORIG_KEY_RANGE = oa.attention_key_range


def _paged_logical_pages(q, k_pages, v_pages, block_table, kv_len, scale):
    n = np.asarray(block_table).shape[1]
    ident = np.tile(np.arange(n), (len(kv_len), 1))
    return ORIG_PAGED(q, k_pages, v_pages, ident, kv_len, scale)          # mistake: table ignored


def _paged_top_left(q, k_pages, v_pages, block_table, kv_len, scale):
    O, L = ORIG_PAGED(q, k_pages, v_pages, block_table, kv_len, scale)
    T_q = np.asarray(q).shape[2]
    if T_q > 1:                                                            # mistake: queries at 0 .. T_q-1
        big = [max(int(n), 1) for n in kv_len]
        O2, L2 = ORIG_PAGED(q, k_pages, v_pages, block_table, [min(T_q, n) for n in big], scale)
        return O2, L2
    return O, L


ORIG_PAGED = oa.paged_attention


MUTATIONS = {
    "top_left_causal": ("visible_keys", _top_left_visible),
    "diagonal_hidden": ("visible_keys", _strict_diagonal),
    "lse_bias": ("_head", _head_no_max_shift),
    "scale_dropped": ("_head", _head_scale_after_softmax),
    "value_transposed": ("_head", _head_transposed_v),
    "head_map_modulo": ("attention", _attention_wrong_head_map),
    "online_no_rescale": ("attention_online", _online_no_rescale),
    "merge_wrong_sign": ("merge_partials", _merge_wrong_sign),
    "partial_off_by_one": ("partial_attention", _partial_off_by_one),
    "key_range_inclusive_end": ("attention_key_range", _key_range_half_open_wrong),
    "key_range_no_causal": ("attention_key_range", _key_range_no_causal),
    "paged_table_ignored": ("paged_attention", _paged_logical_pages),
    "paged_top_left": ("paged_attention", _paged_top_left),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fake = MUTATIONS[name]
    monkeypatch.setattr(oa, attr, fake)
    if hasattr(oracle, attr):
        monkeypatch.setattr(oracle, attr, fake)
    failed = _any_check_fails()
    assert failed, f"no pin caught the planted mistake {name}"

"""Independent checks that pin the float64 oracle to the mathematics.

Each ``check_*`` function raises ``AssertionError`` when the oracle disagrees
with something fixed outside the oracle itself: scalar brute force written
with ``math.fsum``, closed forms, invariants of the definition, or the
hand-derived fixtures in ``tests/golden``.  ``test_oracle_pins.py`` runs them
on the real oracle; ``test_oracle_mutations.py`` plants plausible mistakes in
the oracle and shows that at least one check fails for each.
"""

from __future__ import annotations

import glob
import json
import math
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
_MATH = {"__builtins__": {}, "log": math.log, "exp": math.exp, "sqrt": math.sqrt}


def _num(x):
    if isinstance(x, list):
        return [_num(y) for y in x]
    if isinstance(x, str):
        return float(eval(x, _MATH))  # fixture expressions use math only
    return float(x)


def load_golden(pattern="*.json"):
    out = []
    for path in sorted(glob.glob(os.path.join(GOLDEN, pattern))):
        with open(path) as f:
            fx = json.load(f)
        out.append((os.path.basename(path), {k: (_num(v) if k not in ("cites", "derivation", "causal") else v)
                                             for k, v in fx.items()}))
    return out


# ----------------------------------------------------------------------------
# scalar brute force (no numpy arithmetic)
# ----------------------------------------------------------------------------

def brute_force(q, k, v, scale, causal, kv_len=None):
    """Triple loops over plain Python floats, sums with ``math.fsum``."""
    B, Hq, Sq, d = (len(q), len(q[0]), len(q[0][0]), len(q[0][0][0]))
    Hkv, Skv = len(k[0]), len(k[0][0])
    group = Hq // Hkv
    O = [[[None] * Sq for _ in range(Hq)] for _ in range(B)]
    L = [[[None] * Sq for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        n_keys = Skv if kv_len is None else int(kv_len[b])
        for h in range(Hq):
            kvh = h // group
            for t in range(Sq):
                pos = t + (Skv - Sq)
                keys = [j for j in range(n_keys) if (not causal or j <= pos)]
                if not keys:
                    O[b][h][t] = [0.0] * len(v[b][kvh][0])
                    L[b][h][t] = -math.inf
                    continue
                s = {j: scale * math.fsum(float(q[b][h][t][i]) * float(k[b][kvh][j][i])
                                          for i in range(d)) for j in keys}
                mx = max(s.values())
                w = {j: math.exp(s[j] - mx) for j in keys}
                tot = math.fsum(w.values())
                O[b][h][t] = [math.fsum(w[j] * float(v[b][kvh][j][i]) for j in keys) / tot
                              for i in range(len(v[b][kvh][0]))]
                L[b][h][t] = mx + math.log(tot)
    return np.array(O, dtype=np.float64), np.array(L, dtype=np.float64)


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    err = np.where(both_inf, 0.0, np.abs(a - b))
    assert np.all(np.isfinite(err)), f"{what}: non-finite mismatch"
    m = float(err.max()) if err.size else 0.0
    assert m <= tol, f"{what}: max abs err {m:.3e} > {tol:.1e}"


# ----------------------------------------------------------------------------
# checks
# ----------------------------------------------------------------------------

TINY_SHAPES = [
    # B, Hq, Hkv, Sq, Skv, d
    (1, 1, 1, 1, 1, 1),
    (1, 1, 1, 3, 3, 2),
    (2, 2, 1, 2, 5, 3),
    (1, 4, 2, 4, 4, 4),
    (2, 2, 2, 5, 5, 2),
    (1, 2, 1, 1, 5, 4),
]


def check_brute_force(seed=0):
    """Oracle == scalar brute force on tiny shapes, causal on/off, ragged lengths."""
    r = _rng(seed)
    for (B, Hq, Hkv, Sq, Skv, d) in TINY_SHAPES:
        for causal in (False, True):
            for ragged in (False, True):
                q = r.standard_normal((B, Hq, Sq, d))
                k = r.standard_normal((B, Hkv, Skv, d))
                v = r.standard_normal((B, Hkv, Skv, d))
                scale = float(r.uniform(0.2, 1.5))
                kv_len = r.integers(0, Skv + 1, B) if ragged else None
                if causal and ragged:
                    kv_len = np.maximum(kv_len, 1)
                O, L = oracle.attention(q, k, v, scale, causal, kv_len)
                Ob, Lb = brute_force(q.tolist(), k.tolist(), v.tolist(), scale, causal, kv_len)
                _close(O, Ob, 1e-12, f"O brute {B,Hq,Hkv,Sq,Skv,d} causal={causal}")
                _close(L, Lb, 1e-12, f"LSE brute {B,Hq,Hkv,Sq,Skv,d} causal={causal}")


def check_golden():
    """Oracle reproduces the hand-derived fixtures."""
    for name, fx in load_golden():
        if "q" not in fx:
            continue
        O, L = oracle.attention(np.array(fx["q"]), np.array(fx["k"]), np.array(fx["v"]),
                                fx["scale"], fx["causal"])
        _close(O, np.array(fx["o"]), 1e-12, f"{name} O")
        _close(L, np.array(fx["lse"]), 1e-12, f"{name} LSE")


def check_golden_merge():
    for name, fx in load_golden("merge_*.json"):
        lse, o = oracle.merge_partials(np.array(fx["lse_parts"]), np.array(fx["o_parts"]))
        _close(lse, fx["lse"], 1e-12, f"{name} lse")
        _close(o, np.array(fx["o"]), 1e-12, f"{name} o")


def check_zero_k(seed=1):
    """K = 0: uniform weights, O_t = mean of visible V rows, LSE_t = ln n_t."""
    r = _rng(seed)
    for (Sq, Skv, causal) in [(7, 7, True), (3, 9, True), (6, 6, False), (1, 13, True)]:
        d = 5
        q = r.standard_normal((1, 2, Sq, d))
        k = np.zeros((1, 1, Skv, d))
        v = r.standard_normal((1, 1, Skv, d))
        O, L = oracle.attention(q, k, v, 0.7, causal)
        for t in range(Sq):
            n = (t + 1 + Skv - Sq) if causal else Skv
            _close(O[0, :, t], np.repeat(v[0, 0, :n].mean(axis=0)[None], 2, axis=0), 1e-12,
                   f"zero-K O row {t}")
            _close(L[0, :, t], [math.log(n)] * 2, 1e-12, f"zero-K LSE row {t}")


def check_one_hot(seed=2):
    """K rows are unit vectors; each query picks one visible key with score a*s.

    Closed form: weight e^{a s} on the picked key, weight 1 on every other
    visible key, so O_t = (e^{as} V_pi + sum_{others} V_j) / (e^{as} + n_t - 1)
    and LSE_t = ln(e^{as} + n_t - 1).
    """
    r = _rng(seed)
    d, Skv, Sq = 8, 8, 5
    for causal in (False, True):
        for alpha, scale in [(1024.0, 1 / math.sqrt(128)), (3.0, 0.5), (0.25, 1.0)]:
            k = np.eye(Skv, d)[None, None]
            v = r.standard_normal((1, 1, Skv, d))
            q = np.zeros((1, 1, Sq, d))
            picks = []
            for t in range(Sq):
                n = (t + 1 + Skv - Sq) if causal else Skv
                p = int(r.integers(0, n))
                picks.append((p, n))
                q[0, 0, t, p] = alpha
            O, L = oracle.attention(q, k, v, scale, causal)
            for t, (p, n) in enumerate(picks):
                a = alpha * scale
                # divide through by e^{a} for stability at large a
                others = v[0, 0, :n].sum(axis=0) - v[0, 0, p]
                den = 1.0 + (n - 1) * math.exp(-a)
                exp_o = (v[0, 0, p] + math.exp(-a) * others) / den
                _close(O[0, 0, t], exp_o, 1e-12, f"one-hot O a={alpha} t={t}")
                _close(L[0, 0, t], a + math.log1p((n - 1) * math.exp(-a)), 1e-12,
                       f"one-hot LSE a={alpha} t={t}")


def check_ties(seed=3):
    """c duplicated dominant keys share the weight: O = mean of their V rows,
    LSE = a + ln c (+ the others' negligible e^{-a} mass)."""
    r = _rng(seed)
    d, Skv = 4, 6
    k = np.zeros((1, 1, Skv, d))
    tied = [1, 3, 4]
    for j in tied:
        k[0, 0, j, 0] = 1.0
    v = r.standard_normal((1, 1, Skv, d))
    q = np.zeros((1, 1, 1, d))
    q[0, 0, 0, 0] = 100.0
    O, L = oracle.attention(q, k, v, 1.0, False)
    _close(O[0, 0, 0], v[0, 0, tied].mean(axis=0), 1e-12, "ties O")
    _close(L[0, 0, 0], 100.0 + math.log(3 + 3 * math.exp(-100.0)), 1e-12, "ties LSE")


def check_single_key(seed=4):
    """Skv = 1: O = V_0, LSE = scale * q . k_0."""
    r = _rng(seed)
    q = r.standard_normal((2, 4, 3, 6))
    k = r.standard_normal((2, 2, 1, 6))
    v = r.standard_normal((2, 2, 1, 6))
    O, L = oracle.attention(q, k, v, 0.3, False)
    for b in range(2):
        for h in range(4):
            _close(O[b, h], np.repeat(v[b, h // 2], 3, axis=0), 1e-12, "single-key O")
            _close(L[b, h], 0.3 * q[b, h] @ k[b, h // 2, 0], 1e-12, "single-key LSE")


def check_online_equals_two_pass(seed=5):
    """The pages' tile recurrence equals the two-pass definition for any tile."""
    r = _rng(seed)
    for (B, Hq, Hkv, Sq, Skv, d) in [(1, 2, 1, 9, 9, 4), (2, 4, 2, 5, 17, 3), (1, 1, 1, 1, 11, 2)]:
        q = r.standard_normal((B, Hq, Sq, d)) * 3
        k = r.standard_normal((B, Hkv, Skv, d))
        v = r.standard_normal((B, Hkv, Skv, d))
        for causal in (False, True):
            ref = oracle.attention(q, k, v, 0.9, causal)
            for tile in (1, 3, 4, 64, Skv):
                got = oracle.attention_online(q, k, v, 0.9, causal, tile)
                _close(got[0], ref[0], 1e-12, f"online O tile={tile} causal={causal}")
                _close(got[1], ref[1], 1e-12, f"online LSE tile={tile} causal={causal}")
    # ragged lengths through the recurrence
    q = r.standard_normal((3, 2, 1, 4))
    k = r.standard_normal((3, 1, 10, 4))
    v = r.standard_normal((3, 1, 10, 4))
    lens = np.array([10, 3, 0])
    ref = oracle.attention(q, k, v, 0.5, False, lens)
    got = oracle.attention_online(q, k, v, 0.5, False, 4, lens)
    _close(got[0], ref[0], 1e-12, "online ragged O")
    _close(got[1], ref[1], 1e-12, "online ragged LSE")


def check_merge_any_partition(seed=6):
    """Partials over any contiguous partition, merged in any order or tree,
    give the full decode result (the merge is associative and commutative)."""
    r = _rng(seed)
    Hq, Hkv, S, d = 4, 2, 23, 5
    q = r.standard_normal((Hq, d)) * 2
    k = r.standard_normal((Hkv, S, d))
    v = r.standard_normal((Hkv, S, d))
    O_ref, L_ref = oracle.decode_attention(q[None], k[None], v[None], [S], 0.6)
    for trial in range(12):
        n_cuts = int(r.integers(0, 7))
        cuts = sorted(int(c) for c in r.integers(0, S + 1, n_cuts))
        bounds = [0] + cuts + [S]           # repeated cuts give empty parts
        parts = [oracle.partial_attention(q, k, v, 0.6, lo, hi)
                 for lo, hi in zip(bounds[:-1], bounds[1:])]
        order = r.permutation(len(parts))
        lse = np.stack([parts[i][0] for i in order])
        o = np.stack([parts[i][1] for i in order])
        L, O = oracle.merge_partials(lse, o)
        _close(O, O_ref[0], 1e-12, f"merge order trial {trial}")
        _close(L, L_ref[0], 1e-12, f"merge lse trial {trial}")
        # a different tree: merge the halves first, then the two results
        if len(parts) >= 2:
            h = len(parts) // 2
            La, Oa = oracle.merge_partials(lse[:h], o[:h])
            Lb, Ob = oracle.merge_partials(lse[h:], o[h:])
            L2, O2 = oracle.merge_partials(np.stack([Lb, La]), np.stack([Ob, Oa]))
            _close(O2, O_ref[0], 1e-12, f"merge tree trial {trial}")
            _close(L2, L_ref[0], 1e-12, f"merge tree lse trial {trial}")
    # all parts empty -> (-inf, 0)
    L, O = oracle.merge_partials(np.full((3, Hq), -np.inf), np.zeros((3, Hq, d)))
    assert np.all(np.isneginf(L)) and np.all(O == 0)


def check_gqa_equals_repeated_mha(seed=7):
    """GQA on (Q, K, V) == MHA on K, V repeated G times per KV head."""
    r = _rng(seed)
    for G in (2, 4):
        q = r.standard_normal((2, 2 * G, 6, 3))
        k = r.standard_normal((2, 2, 6, 3))
        v = r.standard_normal((2, 2, 6, 3))
        for causal in (False, True):
            a = oracle.attention(q, k, v, 0.8, causal)
            b = oracle.attention(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), 0.8, causal)
            assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]), "GQA != MHA"


def check_chunked_is_tail(seed=8):
    """A chunk of the last T_q queries over the whole prefix == the last T_q
    rows of the full causal prefill; T_q = 1 == decode over all keys."""
    r = _rng(seed)
    S, d = 12, 4
    q = r.standard_normal((1, 2, S, d))
    k = r.standard_normal((1, 1, S, d))
    v = r.standard_normal((1, 1, S, d))
    full = oracle.attention(q, k, v, 0.5, True)
    for Tq in (1, 3, 5, S):
        ch = oracle.attention(q[:, :, S - Tq:], k, v, 0.5, True)
        _close(ch[0], full[0][:, :, S - Tq:], 1e-13, f"chunk O Tq={Tq}")
        _close(ch[1], full[1][:, :, S - Tq:], 1e-13, f"chunk LSE Tq={Tq}")
    dec = oracle.decode_attention(q[:, :, -1], k, v, [S], 0.5)
    _close(dec[0], full[0][:, :, -1], 1e-13, "decode O == last row")
    _close(dec[1], full[1][:, :, -1], 1e-13, "decode LSE == last row")
    # and the rows of attention_rows agree with the full evaluation
    rows = [0, 5, 11]
    o, l = oracle.attention_rows(q, k, v, 0.5, True, 0, 1, rows)
    _close(o, full[0][0, 1, rows], 1e-13, "attention_rows O")
    _close(l, full[1][0, 1, rows], 1e-13, "attention_rows LSE")


def check_scale_and_permutation(seed=9):
    """(2Q, s/2) == (Q, s); non-causal output invariant under key permutation."""
    r = _rng(seed)
    q = r.standard_normal((1, 2, 5, 4))
    k = r.standard_normal((1, 2, 7, 4))
    v = r.standard_normal((1, 2, 7, 4))
    a = oracle.attention(q, k, v, 0.4, False)
    b = oracle.attention(2 * q, k, v, 0.2, False)
    _close(a[0], b[0], 1e-13, "scale fold O")
    _close(a[1], b[1], 1e-13, "scale fold LSE")
    p = r.permutation(7)
    c = oracle.attention(q, k[:, :, p], v[:, :, p], 0.4, False)
    _close(a[0], c[0], 1e-13, "permutation O")
    _close(a[1], c[1], 1e-13, "permutation LSE")


def check_partial_matches_restricted_definition(seed=10):
    """A split's partial == the definition with only that key range visible."""
    r = _rng(seed)
    q = r.standard_normal((4, 3))
    k = r.standard_normal((2, 10, 3))
    v = r.standard_normal((2, 10, 3))
    for lo, hi in [(0, 10), (2, 7), (9, 10), (4, 4)]:
        L, O = oracle.partial_attention(q, k, v, 1.1, lo, hi)
        if hi <= lo:
            assert np.all(np.isneginf(L)) and np.all(O == 0)
            continue
        Ob, Lb = brute_force(q[None, :, None].tolist(), k[None, :, lo:hi].tolist(),
                             v[None, :, lo:hi].tolist(), 1.1, False)
        _close(O, Ob[0, :, 0], 1e-12, f"partial O {lo}:{hi}")
        _close(L, Lb[0, :, 0], 1e-12, f"partial LSE {lo}:{hi}")


def check_key_range_partials(seed=11):
    """Prefill partials over key ranges: brute force with the range cut out of
    K and V (non-causal; causal via the shifted query block), the full range
    equals the definition, and any partition merged by merge_partials gives
    the full causal GQA result."""
    r = _rng(seed)
    B, Hq, Hkv, Sq, Skv, d = 1, 4, 2, 5, 9, 3
    q = r.standard_normal((B, Hq, Sq, d))
    k = r.standard_normal((B, Hkv, Skv, d))
    v = r.standard_normal((B, Hkv, Skv, d))
    for lo, hi in [(0, Skv), (2, 6), (8, 9), (5, 5)]:
        O, L = oracle.attention_key_range(q, k, v, 0.7, False, lo, hi)
        if hi <= lo:
            assert np.all(np.isneginf(L)) and np.all(O == 0)
            continue
        Ob, Lb = brute_force(q.tolist(), k[:, :, lo:hi].tolist(), v[:, :, lo:hi].tolist(), 0.7, False)
        _close(O, Ob, 1e-12, f"key range O {lo}:{hi}")
        _close(L, Lb, 1e-12, f"key range LSE {lo}:{hi}")
    # causal, range starting at 0: keys [0, hi) for a query block ending at hi
    # is the ordinary causal attention of the rows whose positions are < hi
    full = oracle.attention(q, k, v, 0.7, True)
    same = oracle.attention_key_range(q, k, v, 0.7, True, 0, Skv)
    _close(same[0], full[0], 1e-13, "causal full range O")
    _close(same[1], full[1], 1e-13, "causal full range LSE")
    hi, q_start = 6, Skv - Sq
    part = oracle.attention_key_range(q, k, v, 0.7, True, 0, hi)
    early = [t for t in range(Sq) if q_start + t < hi]    # all their visible keys lie in [0, hi)
    late = [t for t in range(Sq) if q_start + t >= hi]    # they see exactly [0, hi)
    assert early and late
    _close(part[0][:, :, early], full[0][:, :, early], 1e-13, "causal prefix range O (early rows)")
    _close(part[1][:, :, early], full[1][:, :, early], 1e-13, "causal prefix range LSE (early rows)")
    Ob, Lb = brute_force(q[:, :, late].tolist(), k[:, :, :hi].tolist(), v[:, :, :hi].tolist(), 0.7, False)
    _close(part[0][:, :, late], Ob, 1e-12, "causal prefix range O (late rows)")
    _close(part[1][:, :, late], Lb, 1e-12, "causal prefix range LSE (late rows)")
    for trial in range(6):
        cuts = sorted(int(c) for c in r.integers(0, Skv + 1, int(r.integers(0, 5))))
        bounds = [0] + cuts + [Skv]
        parts = [oracle.attention_key_range(q, k, v, 0.7, True, a, b) for a, b in zip(bounds[:-1], bounds[1:])]
        L, O = oracle.merge_partials(np.stack([p[1] for p in parts]), np.stack([p[0] for p in parts]))
        _close(O, full[0], 1e-12, f"key range merge O trial {trial}")
        _close(L, full[1], 1e-12, f"key range merge LSE trial {trial}")


def _pages_from_contiguous(k, page, order):
    """Cut a contiguous cache [B, Hkv, S, d] into pages [B * n_pages, Hkv, page, d]
    placed in the pool at positions given by ``order`` (a permutation); returns
    the pool and the block table that undoes the placement.  Plain slicing."""
    B, Hkv, S, d = k.shape
    n_pages = -(-S // page)
    padded = np.zeros((B, Hkv, n_pages * page, d))
    padded[:, :, :S] = k
    pool = np.zeros((B * n_pages, Hkv, page, d))
    table = np.zeros((B, n_pages), dtype=np.int64)
    for b in range(B):
        for p_ in range(n_pages):
            slot = int(order[b * n_pages + p_])
            pool[slot] = padded[b, :, p_ * page:(p_ + 1) * page]
            table[b, p_] = slot
    return pool, table


def check_paged_attention(seed=12):
    """Multi-token decode over pages: scalar brute force on the gathered keys
    (bottom-right causal within each sequence's valid length), the result does
    not depend on where the pages sit in the pool or on table entries past a
    sequence's last page, and T_q = 1 equals decode_attention."""
    r = _rng(seed)
    B, Hq, Hkv, T_q, S, d, page = 3, 4, 2, 3, 11, 3, 4
    q = r.standard_normal((B, Hq, T_q, d))
    k = r.standard_normal((B, Hkv, S, d))
    v = r.standard_normal((B, Hkv, S, d))
    lens = [11, 5, 2]                        # the last one is shorter than T_q
    order = r.permutation(B * (-(-S // page)))
    kp, table = _pages_from_contiguous(k, page, order)
    vp, _ = _pages_from_contiguous(v, page, order)
    O, L = oracle.paged_attention(q, kp, vp, table, lens, 0.8)
    for b in range(B):
        n = lens[b]
        Ob, Lb = brute_force(q[b:b + 1].tolist(), k[b:b + 1, :, :n].tolist(), v[b:b + 1, :, :n].tolist(), 0.8, True)
        _close(O[b], Ob[0], 1e-12, f"paged O seq {b}")
        _close(L[b], Lb[0], 1e-12, f"paged LSE seq {b}")
    # another placement of the same pages, and garbage past each sequence's pages
    order2 = r.permutation(len(order))
    kp2, table2 = _pages_from_contiguous(k, page, order2)
    vp2, _ = _pages_from_contiguous(v, page, order2)
    for b in range(B):
        used = -(-lens[b] // page)
        table2[b, used:] = r.integers(0, len(order), table2.shape[1] - used)
    O2, L2 = oracle.paged_attention(q, kp2, vp2, table2, lens, 0.8)
    assert np.array_equal(O, O2) and np.array_equal(L, L2), "page placement changed the result"
    # one query token: the decode definition
    O1, L1 = oracle.paged_attention(q[:, :, -1:], kp, vp, table, lens, 0.8)
    kc = np.zeros((B, Hkv, S, d))
    vc = np.zeros((B, Hkv, S, d))
    kc[:], vc[:] = k, v
    Od, Ld = oracle.decode_attention(q[:, :, -1], kc, vc, lens, 0.8)
    _close(O1[:, :, 0], Od, 1e-12, "paged T_q=1 O == decode")
    _close(L1[:, :, 0], Ld, 1e-12, "paged T_q=1 LSE == decode")
    # a sequence without keys
    O0, L0 = oracle.paged_attention(q[:1], kp, vp, table[:1], [0], 0.8)
    assert np.all(O0 == 0) and np.all(np.isneginf(L0))


def check_empty_rows():
    """kv_len = 0 gives O = 0 and LSE = -inf."""
    q = np.ones((2, 2, 1, 3))
    k = np.ones((2, 1, 4, 3))
    v = np.ones((2, 1, 4, 3))
    O, L = oracle.attention(q, k, v, 1.0, False, [0, 4])
    assert np.all(O[0] == 0) and np.all(np.isneginf(L[0]))
    assert np.all(np.isfinite(L[1]))


ALL_CHECKS = [
    check_brute_force, check_golden, check_golden_merge, check_zero_k, check_one_hot,
    check_ties, check_single_key, check_online_equals_two_pass, check_merge_any_partition,
    check_gqa_equals_repeated_mha, check_chunked_is_tail, check_scale_and_permutation,
    check_partial_matches_restricted_definition, check_key_range_partials, check_paged_attention,
    check_empty_rows,
]

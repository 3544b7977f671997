"""attn_decode_splitkv and attn_combine_lse on the GPU against the float64 oracle."""

import math

import numpy as np
import pytest
import torch

import oracle
import streaming_attention_amd as sa
from streaming_attention_amd import workloads as W
from parity import assert_lse, assert_o, f64, split_bounds

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _check_rows(o, lse, q, k, v, lens, scale, seqs, kind="bf16"):
    """Final decode output of the listed sequences, all heads, vs the oracle."""
    for b in seqs:
        n = int(lens[b])
        O_ref, L_ref = oracle.decode_attention(f64(q[b:b + 1, :, 0]), f64(k[b:b + 1, :, :n]),
                                               f64(v[b:b + 1, :, :n]), [n], scale)
        assert_o(o[b, :, 0], O_ref[0], kind, f"O seq {b} len {n}")
        assert_lse(lse[b], L_ref[0], kind, f"LSE seq {b} len {n}")
        # relative error over the heads of this sequence
        num = np.linalg.norm(f64(o[b, :, 0]) - O_ref[0])
        assert num <= 1e-2 * np.linalg.norm(O_ref[0]), f"rel err seq {b}"


def _check_partials(part_o, part_lse, q, k, v, lens, nsplits, scale, seqs, splits=None):
    """Each split's partial vs the oracle restricted to the split's key range."""
    for b in seqs:
        n = int(nsplits[b])
        bounds = split_bounds(int(lens[b]), n)
        which = range(n) if splits is None else [s for s in splits if s < n]
        for s in which:
            lo, hi = bounds[s]
            L_ref, O_ref = oracle.partial_attention(f64(q[b, :, 0]), f64(k[b, :, lo:hi]),
                                                    f64(v[b, :, lo:hi]), scale, 0, hi - lo)
            assert_o(part_o[b, :, s], O_ref, "bf16", f"partial O seq {b} split {s} [{lo},{hi})")
            assert_lse(part_lse[b, :, s], L_ref, "bf16", f"partial LSE seq {b} split {s}")


def _decode_sweep(n, seed):
    """Decode shapes from a seeded generator: batch 1-5, 1-4 KV heads, group
    sizes up to 16, d = 64 or 128, cache capacities that are rarely chunk
    multiples, 1 to 64 split slots, and a seed for the per-sequence lengths
    (0 included) and split counts."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        B, Hkv = int(rng.integers(1, 6)), int(rng.integers(1, 5))
        G = int(rng.choice([1, 2, 4, 5, 8, 16]))
        out.append((B, G * Hkv, Hkv, int(rng.integers(1, 3000)), int(rng.choice([64, 128])),
                    int(rng.choice([1, 3, 8, 17, 64])), int(rng.integers(0, 1 << 30))))
    return out


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("B,Hq,Hkv,S_cap,d,max_splits,seed", _decode_sweep(16, 91))
def test_decode_seeded_sweep(B, Hq, Hkv, S_cap, d, max_splits, seed, fused):
    """Random decode shapes, per-sequence lengths (some 0) and split counts,
    split + merge and the one-launch form: every sequence and head against
    the oracle."""
    rng = np.random.default_rng(seed)
    lens = [int(x) for x in rng.integers(0, S_cap + 1, B)]
    if B > 1:
        lens[int(rng.integers(0, B))] = S_cap
    ns = [int(x) for x in rng.integers(1, max_splits + 1, B)]
    g = torch.Generator(device=DEV).manual_seed(seed % 100000)
    q = torch.randn((B, Hq, 1, d), generator=g, device=DEV).to(torch.bfloat16)
    k = torch.randn((B, Hkv, S_cap, d), generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn((B, Hkv, S_cap, d), generator=g, device=DEV).to(torch.bfloat16)
    kv_len = torch.tensor(lens, dtype=torch.int32, device=DEV)
    nsp = torch.tensor(ns, dtype=torch.int32, device=DEV)
    scale = 1 / math.sqrt(d)
    o, lse = sa.decode(q, k, v, kv_len, nsp, max_splits=max_splits, scale=scale, fused=fused)
    torch.cuda.synchronize()
    _check_rows(o, lse, q, k, v, lens, scale, range(B))


def test_gqa70b_decode_full_size():
    """B=4, 64/8 heads, 32768 keys each, 64 splits: every output row and a
    sample of split partials, in the benchmark's launch shape."""
    w = W.GQA70B_DECODE
    q, k, v, lens = W.decode_inputs(w, DEV)
    part_o, part_lse = sa.decode_splitkv(q, k, v, None, None, max_splits=w.splits, scale=w.scale)
    o, lse = sa.combine_lse(part_o, part_lse, None, torch.bfloat16)
    torch.cuda.synchronize()
    _check_rows(o, lse, q, k, v, lens, w.scale, range(w.B))
    ns = [w.splits] * w.B
    _check_partials(part_o, part_lse, q, k, v, lens, ns, w.scale, [0, 3], splits=[0, 1, 31, 63])


@pytest.fixture(scope="module")
def ragged():
    """The ragged decode workload (B=16, lengths uniform in [1024, 131072]
    from the seed, NaN past every length) and the oracle's result for every
    sequence, computed once for the tests that share it."""
    w = W.RAGGED_DECODE
    q, k, v, lens = W.decode_inputs(w, DEV)
    ref = {}
    for b in range(w.B):
        n = int(lens[b])
        ref[b] = oracle.decode_attention(f64(q[b:b + 1, :, 0]), f64(k[b:b + 1, :, :n]), f64(v[b:b + 1, :, :n]),
                                         [n], w.scale)
    return w, q, k, v, lens, ref


def _check_all_sequences(o, lse, ragged):
    w, q, k, v, lens, ref = ragged
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all(), "an output was not written"
    for b in range(w.B):
        O_ref, L_ref = ref[b]
        n = int(lens[b])
        assert_o(o[b, :, 0], O_ref[0], "bf16", f"O seq {b} len {n}")
        assert_lse(lse[b], L_ref[0], "bf16", f"LSE seq {b} len {n}")
        num = np.linalg.norm(f64(o[b, :, 0]) - O_ref[0])
        assert num <= 1e-2 * np.linalg.norm(O_ref[0]), f"rel err seq {b}"


def _nan_out(w):
    o = torch.full((w.B, w.Hq, 1, w.d), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((w.B, w.Hq), float("nan"), dtype=torch.float32, device=DEV)
    return o, lse


def test_ragged_decode_full_size_every_sequence(ragged):
    """Split count per length, split + merge in two launches (the launch the
    benchmark times): outputs start as NaN; all 16 sequences meet the bar."""
    w, q, k, v, lens, _ = ragged
    ns = sa.splits_for_lengths(lens)
    o, lse = _nan_out(w)
    sa.decode(q, k, v, lens.to(DEV), ns.to(DEV), max_splits=64, scale=w.scale, fused=False, out=o, lse=lse)
    torch.cuda.synchronize()
    _check_all_sequences(o, lse, ragged)


SMALL = [
    # B, Hq, Hkv, S_cap, d, lens, nsplits, max_splits
    (3, 8, 1, 700, 128, [700, 1, 333], [4, 1, 3], 4),
    (2, 16, 2, 1000, 64, [1000, 64], [7, 7], 8),
    (4, 4, 4, 300, 128, [0, 5, 299, 300], [2, 3, 1, 5], 5),
    (2, 32, 2, 129, 128, [129, 128], [256, 3], 256),
    (1, 64, 8, 4096, 128, [4095], [64], 64),
    (2, 2, 2, 97, 64, [97, 96], [1, 2], 2),
]


@pytest.mark.parametrize("B,Hq,Hkv,S_cap,d,lens,nsplits,max_splits", SMALL)
def test_small_decode_with_partials(B, Hq, Hkv, S_cap, d, lens, nsplits, max_splits):
    g = torch.Generator(device=DEV).manual_seed(77 + S_cap + d)
    q = torch.randn((B, Hq, 1, d), generator=g, device=DEV).to(torch.bfloat16)
    k = torch.randn((B, Hkv, S_cap, d), generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn((B, Hkv, S_cap, d), generator=g, device=DEV).to(torch.bfloat16)
    for b, n in enumerate(lens):       # poison everything past each length
        k[b, :, n:] = float("nan")
        v[b, :, n:] = float("nan")
    lt = torch.tensor(lens, dtype=torch.int32, device=DEV)
    nt = torch.tensor(nsplits, dtype=torch.int32, device=DEV)
    scale = 1 / math.sqrt(d)
    part_o, part_lse = sa.decode_splitkv(q, k, v, lt, nt, max_splits=max_splits, scale=scale)
    o, lse = sa.combine_lse(part_o, part_lse, nt, torch.bfloat16)
    torch.cuda.synchronize()
    for b in range(B):
        n = lens[b]
        if n == 0:
            assert (o[b].float() == 0).all() and torch.isneginf(lse[b]).all()
            continue
        O_ref, L_ref = oracle.decode_attention(f64(q[b:b + 1, :, 0]), f64(k[b:b + 1, :, :n]),
                                               f64(v[b:b + 1, :, :n]), [n], scale)
        assert_o(o[b, :, 0], O_ref[0], "bf16")
        assert_lse(lse[b], L_ref[0], "bf16")
    _check_partials(part_o, part_lse, q, k, v, lens, nsplits, scale, range(B))


def test_default_lengths_and_splits():
    """kv_len = NULL means S_cap keys; num_splits = NULL means max_splits."""
    B, Hq, Hkv, S, d = 2, 8, 1, 517, 128
    q = torch.randn(B, Hq, 1, d, device=DEV).to(torch.bfloat16)
    k = torch.randn(B, Hkv, S, d, device=DEV).to(torch.bfloat16)
    v = torch.randn(B, Hkv, S, d, device=DEV).to(torch.bfloat16)
    o, lse = sa.decode(q, k, v, max_splits=6)
    torch.cuda.synchronize()
    _check_rows(o, lse, q, k, v, [S] * B, 1 / math.sqrt(d), range(B))


def test_combine_fp32_output_and_random_partials():
    """The combine kernel alone on arbitrary partials (including -inf entries)
    against the oracle's log-sum-exp merge; fp32 output at 1e-4."""
    rng = np.random.default_rng(3)
    B, Hq, S, d = 3, 5, 9, 64
    lse_p = rng.normal(0.0, 3.0, (B, Hq, S))
    lse_p[0, 0, :4] = -np.inf
    lse_p[2, :, :] = -np.inf              # a sequence with nothing to attend
    o_p = rng.standard_normal((B, Hq, S, d))
    po = torch.tensor(o_p, dtype=torch.float32, device=DEV)
    pl = torch.tensor(lse_p, dtype=torch.float32, device=DEV)
    ns = torch.tensor([9, 4, 9], dtype=torch.int32, device=DEV)
    o, lse = sa.combine_lse(po, pl, ns, torch.float32)
    torch.cuda.synchronize()
    for b in range(B):
        n = int(ns[b])
        L_ref, O_ref = oracle.merge_partials(np.moveaxis(f64(pl[b, :, :n]), 1, 0),
                                             np.moveaxis(f64(po[b, :, :n]), 1, 0))
        assert_o(o[b, :, 0], O_ref, "f32")
        assert_lse(lse[b], L_ref, "f32")


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_combine_few_splits_per_sequence_counts(d, out_dtype):
    """The merge for at most 8 splits (one wave per row) on arbitrary partials:
    per-sequence counts 1..8 out of 8 slots, -inf entries, a row with every
    split empty; against the oracle's log-sum-exp merge of the first n_b
    slots (slots past n_b hold values that must not count)."""
    rng = np.random.default_rng(11 + d)
    B, Hq, S = 9, 6, 8
    lse_p = rng.normal(0.0, 3.0, (B, Hq, S))
    lse_p[1, 2, :3] = -np.inf
    lse_p[4, 0, :] = -np.inf
    o_p = rng.standard_normal((B, Hq, S, d))
    po = torch.tensor(o_p, dtype=torch.float32, device=DEV)
    pl = torch.tensor(lse_p, dtype=torch.float32, device=DEV)
    counts = [1, 2, 3, 4, 5, 6, 7, 8, 8]
    ns = torch.tensor(counts, dtype=torch.int32, device=DEV)
    o, lse = sa.combine_lse(po, pl, ns, out_dtype)
    torch.cuda.synchronize()
    kind = "f32" if out_dtype == torch.float32 else "bf16"
    for b in range(B):
        n = counts[b]
        L_ref, O_ref = oracle.merge_partials(np.moveaxis(f64(pl[b, :, :n]), 1, 0),
                                             np.moveaxis(f64(po[b, :, :n]), 1, 0))
        assert_o(o[b, :, 0], O_ref, kind)
        assert_lse(lse[b], L_ref, "f32")


def test_decode_matches_last_row_of_prefill_oracle():
    """Decode over len keys == the last row of a causal prefill over them."""
    S, d = 1500, 128
    q = torch.randn(1, 8, S, d, device=DEV).to(torch.bfloat16)
    k = torch.randn(1, 1, S, d, device=DEV).to(torch.bfloat16)
    v = torch.randn(1, 1, S, d, device=DEV).to(torch.bfloat16)
    o, lse = sa.decode(q[:, :, -1:].contiguous(), k, v, max_splits=7)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention_rows(f64(q[:, :8]), f64(k), f64(v), 1 / math.sqrt(d), True, 0, 0, [S - 1])
    assert_o(o[0, 0, 0], O_ref[0], "bf16")
    assert_lse(lse[0, 0], L_ref[0], "bf16")


def test_decode_repeat_is_bitwise():
    w = W.GQA70B_DECODE
    q, k, v, _ = W.decode_inputs(w, DEV, B=1, S_cap=8192)
    o1, l1 = sa.decode(q, k, v, max_splits=16)
    o2, l2 = sa.decode(q, k, v, max_splits=16)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ---------------------------------------------------------------------------
# attn_decode: split-KV + merge in one launch
# ---------------------------------------------------------------------------

def test_fused_decode_full_size_and_counters_reset():
    """The 70B-shape decode through the fused entry point (the launch the bench
    times), three calls in a row on one counter buffer."""
    w = W.GQA70B_DECODE
    q, k, v, lens = W.decode_inputs(w, DEV)
    cnt = torch.zeros(w.B * w.Hkv, dtype=torch.int32, device=DEV)
    for _ in range(3):
        o, lse = sa.decode(q, k, v, None, None, max_splits=w.splits, scale=w.scale, counters=cnt, fused=True)
    torch.cuda.synchronize()
    assert int(cnt.abs().sum()) == 0, "counters must be zero after the launch"
    _check_rows(o, lse, q, k, v, lens, w.scale, range(w.B))


def test_fused_decode_ragged_every_sequence(ragged):
    w, q, k, v, lens, _ = ragged
    ns = sa.splits_for_lengths(lens)
    o, lse = _nan_out(w)
    sa.decode(q, k, v, lens.to(DEV), ns.to(DEV), max_splits=64, scale=w.scale, fused=True, out=o, lse=lse)
    torch.cuda.synchronize()
    _check_all_sequences(o, lse, ragged)


@pytest.mark.parametrize("B,Hq,Hkv,S_cap,d,lens,nsplits,max_splits", SMALL)
def test_fused_small_decode(B, Hq, Hkv, S_cap, d, lens, nsplits, max_splits):
    g = torch.Generator(device=DEV).manual_seed(99 + S_cap + d)
    q = torch.randn((B, Hq, 1, d), generator=g, device=DEV).to(torch.bfloat16)
    k = torch.randn((B, Hkv, S_cap, d), generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn((B, Hkv, S_cap, d), generator=g, device=DEV).to(torch.bfloat16)
    for b, n in enumerate(lens):
        k[b, :, n:] = float("nan")
        v[b, :, n:] = float("nan")
    lt = torch.tensor(lens, dtype=torch.int32, device=DEV)
    nt = torch.tensor(nsplits, dtype=torch.int32, device=DEV)
    scale = 1 / math.sqrt(d)
    o, lse = sa.decode(q, k, v, lt, nt, max_splits=max_splits, scale=scale, fused=True)
    torch.cuda.synchronize()
    for b in range(B):
        n = lens[b]
        if n == 0:
            assert (o[b].float() == 0).all() and torch.isneginf(lse[b]).all()
            continue
        O_ref, L_ref = oracle.decode_attention(f64(q[b:b + 1, :, 0]), f64(k[b:b + 1, :, :n]),
                                               f64(v[b:b + 1, :, :n]), [n], scale)
        assert_o(o[b, :, 0], O_ref[0], "bf16")
        assert_lse(lse[b], L_ref[0], "bf16")


def test_out_of_range_lengths_and_split_counts_are_clamped():
    """kv_len and num_splits are device data the host cannot check: lengths
    act as clamped to [0, S_cap], split counts to [1, max_splits]."""
    B, Hq, Hkv, S_cap, d, max_splits = 4, 8, 2, 300, 128, 4
    g = torch.Generator(device=DEV).manual_seed(4242)
    q = torch.randn((B, Hq, 1, d), generator=g, device=DEV).to(torch.bfloat16)
    k = torch.randn((B, Hkv, S_cap, d), generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn((B, Hkv, S_cap, d), generator=g, device=DEV).to(torch.bfloat16)
    lens = torch.tensor([-5, S_cap + 100, 10, 299], dtype=torch.int32, device=DEV)
    ns = torch.tensor([0, 999, 2, -3], dtype=torch.int32, device=DEV)
    scale = 1 / math.sqrt(d)
    o, lse = sa.decode(q, k, v, lens, ns, max_splits, scale=scale)
    torch.cuda.synchronize()
    _check_rows(o, lse, q, k, v, [0, S_cap, 10, 299], scale, range(B))

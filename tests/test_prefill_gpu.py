"""attn_prefill on the GPU against the float64 oracle."""

import math

import numpy as np
import pytest
import torch

import oracle
import streaming_attention_amd as sa
from streaming_attention_amd import workloads as W
from parity import (assert_lse, assert_o, assert_rel_fro, block_rows, check_prefill_rows, f64, nan_outputs,
                    prefill_split_bounds)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _kind(t):
    return "bf16" if t.dtype == torch.bfloat16 else "f32"


def run_and_check(q, k, v, causal, scale=None, rel_fro=True):
    d = q.shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    o, lse = sa.prefill(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention(f64(q), f64(k), f64(v), scale, causal)
    kind = _kind(q)
    assert_o(o, O_ref, kind)
    assert_lse(lse, L_ref, kind)
    if kind == "bf16" and rel_fro:
        assert_rel_fro(o, O_ref)
    return o, lse


def test_single_head_f32_full():
    """fp32, B=1, H=1, S=128, d=64, non-causal: the whole output at 1e-4."""
    w = W.SINGLE_HEAD_F32
    q, k, v = W.prefill_inputs(w, DEV)
    run_and_check(q, k, v, w.causal, w.scale)


def test_mha_causal_prefill_full():
    """bf16, B=2, H=16, S=1024, d=64, causal: the whole output."""
    w = W.MHA_CAUSAL
    q, k, v = W.prefill_inputs(w, DEV)
    run_and_check(q, k, v, w.causal, w.scale)


# Small shapes that span several tiles, ragged tails, GQA rows of two heads in
# one 128-row tile, d = 64 and 128, causal on and off, bf16 and fp32.
SMALL = [
    # B, Hq, Hkv, Sq, Skv, d, causal, dtype
    (1, 8, 1, 200, 333, 128, False, torch.bfloat16),
    (2, 4, 2, 77, 300, 64, True, torch.bfloat16),
    (1, 16, 2, 130, 130, 128, True, torch.bfloat16),
    (1, 8, 8, 1, 257, 128, True, torch.bfloat16),
    (2, 6, 3, 96, 96, 64, False, torch.bfloat16),
    (1, 2, 1, 65, 65, 128, True, torch.float32),
    (1, 4, 2, 100, 190, 64, True, torch.float32),
    (2, 2, 2, 33, 31, 128, False, torch.float32),
    (1, 1, 1, 1, 1, 64, True, torch.bfloat16),
    (1, 32, 8, 48, 1000, 128, True, torch.bfloat16),
]


@pytest.mark.parametrize("B,Hq,Hkv,Sq,Skv,d,causal,dtype", SMALL)
def test_small_shapes(B, Hq, Hkv, Sq, Skv, d, causal, dtype):
    g = torch.Generator(device=DEV).manual_seed(1000 + Sq + Skv + d)
    q = torch.randn((B, Hq, Sq, d), generator=g, device=DEV).to(dtype)
    k = torch.randn((B, Hkv, Skv, d), generator=g, device=DEV).to(dtype)
    v = torch.randn((B, Hkv, Skv, d), generator=g, device=DEV).to(dtype)
    run_and_check(q, k, v, causal)


def _sweep_shapes(n, seed, large=False):
    """Shapes drawn from a seeded generator: batch 1-2, 1-3 KV heads (8 for the
    large ones), group sizes 1, 2, 4, 5 or 8, d = 64 or 128, causal or not,
    lengths that are rarely tile multiples.  Large shapes give at least 256
    workgroups of 256 rows, so the 8-wave (two-team) launch runs."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        d = int(rng.choice([64, 128]))
        causal = bool(rng.integers(0, 2))
        if large:
            B, Hkv, G = int(rng.integers(1, 3)), 8, int(rng.choice([1, 4, 8]))
            Sq = int(rng.integers(600, 1400))
            if -(-G * Sq // 256) * B * Hkv < 256:
                continue
            Skv = int(rng.integers(Sq if causal else 300, 1600))
        else:
            B, Hkv, G = int(rng.integers(1, 3)), int(rng.choice([1, 2, 3])), int(rng.choice([1, 2, 4, 5, 8]))
            Sq = int(rng.integers(1, 260))
            Skv = int(rng.integers(Sq if causal else 1, 520))
        out.append((B, G * Hkv, Hkv, Sq, Skv, d, causal))
    return out


@pytest.mark.parametrize("B,Hq,Hkv,Sq,Skv,d,causal", _sweep_shapes(40, 77))
def test_seeded_shape_sweep(B, Hq, Hkv, Sq, Skv, d, causal):
    """Random shapes of the default launch, every output element against the
    oracle; every third shape also through two or three key splits and the
    merge."""
    g = torch.Generator(device=DEV).manual_seed(5000 + B * 7 + Hq * 13 + Sq + 3 * Skv + d)
    q = torch.randn((B, Hq, Sq, d), generator=g, device=DEV).to(torch.bfloat16)
    k = torch.randn((B, Hkv, Skv, d), generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn((B, Hkv, Skv, d), generator=g, device=DEV).to(torch.bfloat16)
    o, lse = run_and_check(q, k, v, causal)
    if (Sq + Skv) % 3 == 0:
        n = 2 + (Sq + Skv) % 2
        o2, lse2 = sa.prefill(q, k, v, causal=causal, num_splits=n)
        torch.cuda.synchronize()
        O_ref, L_ref = oracle.attention(f64(q), f64(k), f64(v), 1.0 / math.sqrt(d), causal)
        assert_o(o2, O_ref, "bf16", f"O ({n} splits)")
        assert_lse(lse2, L_ref, "bf16", f"LSE ({n} splits)")


@pytest.mark.parametrize("B,Hq,Hkv,Sq,Skv,d,causal", _sweep_shapes(10, 79))
def test_seeded_shape_sweep_f32(B, Hq, Hkv, Sq, Skv, d, causal):
    """Random shapes on the fp32 path, every output element at 1e-4."""
    g = torch.Generator(device=DEV).manual_seed(7000 + B * 7 + Hq * 13 + Sq + 3 * Skv + d)
    q = torch.randn((B, Hq, Sq, d), generator=g, device=DEV)
    k = torch.randn((B, Hkv, Skv, d), generator=g, device=DEV)
    v = torch.randn((B, Hkv, Skv, d), generator=g, device=DEV)
    run_and_check(q, k, v, causal)


@pytest.mark.parametrize("B,Hq,Hkv,Sq,Skv,d,causal", _sweep_shapes(10, 78, large=True))
def test_seeded_shape_sweep_eight_wave(B, Hq, Hkv, Sq, Skv, d, causal):
    """Random shapes of the 8-wave launch: outputs start as NaN and must all be
    written; one row of every 32-position block of every head against the
    oracle."""
    g = torch.Generator(device=DEV).manual_seed(6000 + B * 7 + Hq * 13 + Sq + 3 * Skv + d)
    q = torch.randn((B, Hq, Sq, d), generator=g, device=DEV).to(torch.bfloat16)
    k = torch.randn((B, Hkv, Skv, d), generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn((B, Hkv, Skv, d), generator=g, device=DEV).to(torch.bfloat16)
    scale = 1.0 / math.sqrt(d)
    o, lse = nan_outputs(q)
    sa.prefill(q, k, v, causal=causal, scale=scale, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all(), "an output row was not written"
    rows = sorted(r for r in set(block_rows(Sq, np.random.default_rng(Sq + Skv), block=32)) | {0, Sq - 1})
    check_prefill_rows(o, lse, q, k, v, scale, causal, rows)


def _full_size_check(w, per_block, num_splits=None, block=32):
    """The workload at full size, in the launch the benchmark times: outputs
    start as NaN and must be finite everywhere afterwards (every M tile
    written), and in every query head ``per_block`` random rows of each
    ``block``-position block meet the bar against the oracle, with the
    relative Frobenius guard over the checked rows of each 128-row block.
    With G = 8 a workgroup of the 8-wave launch holds 32 positions of the 8
    query heads of a KV head, so 32-position blocks check every workgroup's
    rows in every head."""
    q, k, v = W.prefill_inputs(w, DEV)
    o, lse = nan_outputs(q)
    sa.prefill(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse, num_splits=num_splits)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all(), "an output row was not written"
    rows = block_rows(w.Sq, np.random.default_rng(w.seed), block=block, per_block=per_block)
    return check_prefill_rows(o, lse, q, k, v, w.scale, w.causal, rows, what=f" {w.name}")


def test_gqa70b_prefill_full_size_rows_of_every_tile():
    """B=1, 64/8 heads, S=8192, d=128, causal: one row of every 32-position
    block of all 64 heads (16,448 rows) against the oracle."""
    _full_size_check(W.GQA70B_PREFILL, per_block=1)


def test_chunked_prefill_full_size_rows_of_every_tile():
    """512 new queries over a 65536-token prefix (bottom-right causal), in the
    default split-KV launch and unsplit: two rows of every 32-position block
    of all 64 heads."""
    w = W.CHUNKED_PREFILL
    assert sa.prefill_splits(w.B, w.Hq, w.Hkv, w.Sq, w.Skv) == 2
    _full_size_check(w, per_block=2)
    _full_size_check(w, per_block=2, num_splits=1)


def test_skv_zero_noncausal_gives_zero_and_neg_inf():
    q = torch.randn(1, 2, 5, 64, device=DEV).to(torch.bfloat16)
    k = torch.empty(1, 1, 0, 64, device=DEV, dtype=torch.bfloat16)
    o, lse = sa.prefill(q, k, k, causal=False)
    torch.cuda.synchronize()
    assert (o.float() == 0).all() and torch.isneginf(lse).all()


def test_empty_query_block_is_a_noop():
    q = torch.empty(1, 2, 0, 128, device=DEV, dtype=torch.bfloat16)
    k = torch.randn(1, 1, 9, 128, device=DEV).to(torch.bfloat16)
    o, lse = sa.prefill(q, k, k, causal=True)
    assert o.shape == (1, 2, 0, 128) and lse.shape == (1, 2, 0)


def test_zero_k_gives_running_mean_of_v():
    """K = 0: uniform weights, O_t = mean of visible V rows, LSE_t = ln n_t."""
    Sq = Skv = 300
    q = torch.randn(1, 4, Sq, 128, device=DEV).to(torch.bfloat16)
    k = torch.zeros(1, 2, Skv, 128, device=DEV, dtype=torch.bfloat16)
    v = torch.randn(1, 2, Skv, 128, device=DEV).to(torch.bfloat16)
    o, lse = sa.prefill(q, k, v, causal=True)
    torch.cuda.synchronize()
    vv = f64(v)
    n = np.arange(1, Sq + 1)
    mean = np.cumsum(vv, axis=2) / n[None, None, :, None]
    ref = np.repeat(mean, 2, axis=1)
    assert_o(o, ref, "bf16")
    assert_lse(lse, np.broadcast_to(np.log(n), (1, 4, Sq)), "bf16")


def test_one_hot_scores_select_one_value_row():
    """K rows are unit vectors; query t puts 1024 on coordinate pi(t) <= t, so
    softmax saturates on key pi(t): O_t = V_pi(t), LSE_t = 1024 * scale (+ tiny)."""
    S, d = 128, 128
    scale = 1.0 / math.sqrt(d)
    k = torch.eye(S, d, device=DEV).to(torch.bfloat16)[None, None]
    rng = np.random.default_rng(5)
    pick = [int(rng.integers(0, t + 1)) for t in range(S)]
    q = torch.zeros(1, 1, S, d, device=DEV)
    for t, p in enumerate(pick):
        q[0, 0, t, p] = 1024.0
    q = q.to(torch.bfloat16)
    v = torch.randn(1, 1, S, d, device=DEV).to(torch.bfloat16)
    o, lse = sa.prefill(q, k, v, causal=True, scale=scale)
    torch.cuda.synchronize()
    ref = f64(v)[0, 0, pick]
    assert_o(o[0, 0], ref, "bf16")
    a = 1024.0 * scale
    lse_ref = [a + math.log1p(t * math.exp(-a)) for t in range(S)]
    assert_lse(lse[0, 0], lse_ref, "bf16")


def test_scale_folding_is_bitwise():
    """(2Q, scale/2) and (Q, scale) give bitwise-identical outputs: doubling a
    bf16 value and halving the fp32 scale are both exact."""
    q = torch.randn(1, 8, 256, 128, device=DEV).to(torch.bfloat16)
    k = torch.randn(1, 2, 256, 128, device=DEV).to(torch.bfloat16)
    v = torch.randn(1, 2, 256, 128, device=DEV).to(torch.bfloat16)
    o1, l1 = sa.prefill(q, k, v, causal=True, scale=0.125)
    o2, l2 = sa.prefill(q * 2, k, v, causal=True, scale=0.0625)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_repeat_runs_are_bitwise_identical():
    w = W.MHA_CAUSAL
    q, k, v = W.prefill_inputs(w, DEV)
    o1, l1 = sa.prefill(q, k, v, causal=True)
    o2, l2 = sa.prefill(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_gqa_and_repeated_mha_both_match_the_oracle():
    """The same attention as GQA (8 query heads per KV head) and as MHA on
    repeat-interleaved K/V: both launches against the one GQA oracle result."""
    q = torch.randn(1, 16, 200, 128, device=DEV).to(torch.bfloat16)
    k = torch.randn(1, 2, 200, 128, device=DEV).to(torch.bfloat16)
    v = torch.randn(1, 2, 200, 128, device=DEV).to(torch.bfloat16)
    O_ref, L_ref = oracle.attention(f64(q), f64(k), f64(v), 1 / math.sqrt(128), True)
    o1, l1 = sa.prefill(q, k, v, causal=True)
    kr = k.repeat_interleave(8, dim=1).contiguous()
    vr = v.repeat_interleave(8, dim=1).contiguous()
    o2, l2 = sa.prefill(q, kr, vr, causal=True)
    torch.cuda.synchronize()
    for o, l in ((o1, l1), (o2, l2)):
        assert_o(o, O_ref, "bf16")
        assert_lse(l, L_ref, "bf16")


def test_nan_after_the_last_key_row_is_never_read():
    """Keys past Skv are never read: K and V are views at the front of larger
    NaN-filled buffers, so the bytes right after their last row are NaN."""
    Skv, shape = 100, (1, 2, 100, 128)
    n = 1 * 2 * Skv * 128
    kbuf = torch.full((n + 64 * 128,), float("nan"), device=DEV, dtype=torch.bfloat16)
    vbuf = torch.full_like(kbuf, float("nan"))
    k = kbuf[:n].view(shape)
    v = vbuf[:n].view(shape)
    k.copy_(torch.randn(shape, device=DEV).to(torch.bfloat16))
    v.copy_(torch.randn(shape, device=DEV).to(torch.bfloat16))
    q = torch.randn(1, 4, 70, 128, device=DEV).to(torch.bfloat16)
    run_and_check(q, k, v, causal=True)


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("step", [2.0, 0.3, -1.0])
def test_scores_that_climb_or_fall_across_tiles(step, causal, d):
    """Key rows drift along the query direction by `step` per 64-key tile, so
    the scores of later tiles rise far above (step 2.0: about 32 log2 units a
    tile), gently above (0.3: the exponent base is raised only after several
    tiles) or fall below (-1.0) the first tile's maximum.  Every kernel choice
    of exponent base must still give the exact softmax."""
    g = torch.Generator(device=DEV).manual_seed(int(100 * step) + d + causal)
    Sq, Skv = 100, 600
    q = (1.0 + 0.25 * torch.randn((1, 2, Sq, d), generator=g, device=DEV)).to(torch.bfloat16)
    drift = step * (torch.arange(Skv, device=DEV) // 64).float()
    k = (drift[None, None, :, None] + 0.25 * torch.randn((1, 1, Skv, d), generator=g, device=DEV)).to(torch.bfloat16)
    v = torch.randn((1, 1, Skv, d), generator=g, device=DEV).to(torch.bfloat16)
    o, lse = run_and_check(q, k, v, causal)
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()



# Split-KV prefill: every split's partial against the definition restricted to
# its key range, and the merged result against the whole definition.  Cases:
# GQA causal chunk after a prefix, non-causal d = 64, many splits of a short
# query block, more splits than tiles (empty splits), a single query row.
SPLIT = [
    # B, Hq, Hkv, Sq, Skv, d, causal, n
    (1, 8, 2, 130, 700, 128, True, 3),
    (2, 4, 4, 64, 333, 64, False, 4),
    (1, 16, 2, 40, 1000, 128, True, 7),
    (1, 2, 1, 16, 100, 128, True, 5),
    (1, 8, 8, 1, 257, 128, True, 2),
]


@pytest.mark.parametrize("B,Hq,Hkv,Sq,Skv,d,causal,n", SPLIT)
def test_split_prefill_partials_and_merge(B, Hq, Hkv, Sq, Skv, d, causal, n):
    g = torch.Generator(device=DEV).manual_seed(2000 + Sq + Skv + n)
    q = torch.randn((B, Hq, Sq, d), generator=g, device=DEV).to(torch.bfloat16)
    k = torch.randn((B, Hkv, Skv, d), generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn((B, Hkv, Skv, d), generator=g, device=DEV).to(torch.bfloat16)
    scale = 1.0 / math.sqrt(d)
    po, pl = sa.prefill_splitkv(q, k, v, n, causal=causal, scale=scale)
    o, lse = sa.prefill(q, k, v, causal=causal, scale=scale, num_splits=n)
    torch.cuda.synchronize()
    qf, kf, vf = f64(q), f64(k), f64(v)
    for s, (lo, hi) in enumerate(prefill_split_bounds(Skv, n)):
        O_s, L_s = oracle.attention_key_range(qf, kf, vf, scale, causal, lo, hi)
        assert_o(po[:, :, :, s], O_s, "bf16", f"partial O split {s} [{lo},{hi})")
        assert_lse(pl[:, :, :, s], L_s, "bf16", f"partial LSE split {s} [{lo},{hi})")
    O_ref, L_ref = oracle.attention(qf, kf, vf, scale, causal)
    assert_o(o, O_ref, "bf16")
    assert_lse(lse, L_ref, "bf16")
    assert_rel_fro(o, O_ref)


def test_split_prefill_without_keys_gives_zero_and_neg_inf():
    q = torch.randn(1, 4, 8, 128, device=DEV).to(torch.bfloat16)
    k = torch.empty(1, 2, 0, 128, device=DEV, dtype=torch.bfloat16)
    po, pl = sa.prefill_splitkv(q, k, k, 3, causal=False)
    o, lse = sa.prefill(q, k, k, causal=False, num_splits=3)
    torch.cuda.synchronize()
    assert torch.all(po == 0) and torch.all(torch.isneginf(pl))
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


# Shapes large enough for the 8-wave (256-row) workgroups, d = 64 and 128,
# causal and not, checked on one sampled row of every 32-position block of
# every head (the small shapes above run the 4-wave launch).  With G a
# multiple of 8 a workgroup is 32 positions of 8 query heads, otherwise 256
# consecutive stacked rows.
EIGHT_WAVE = [
    # B, Hq, Hkv, Sq, Skv, d, causal
    (1, 32, 32, 2048, 2048, 64, False),
    (1, 64, 8, 1024, 1500, 128, False),
    (2, 16, 2, 2048, 2048, 64, True),
    (2, 40, 8, 1000, 1000, 128, True),     # G = 5: row blocks straddle query heads, ragged last block
    (2, 64, 4, 1000, 1000, 128, True),     # G = 16: two blocks of 8 heads per KV head, ragged last positions
    (2, 32, 4, 1000, 1300, 64, True),      # G = 8, d = 64: ragged last positions, queries after a 300-key prefix
    (32, 64, 8, 20, 20, 128, True),        # G = 8, one partial 32-position block (20 rows per wave)
    (1, 96, 4, 700, 700, 128, True),       # G = 24: three blocks of 8 heads per KV head, ragged last positions
]


@pytest.mark.parametrize("B,Hq,Hkv,Sq,Skv,d,causal", EIGHT_WAVE)
def test_eight_wave_launch_rows_of_every_tile(B, Hq, Hkv, Sq, Skv, d, causal):
    assert -(-(Hq // Hkv) * Sq // 256) * B * Hkv >= 256      # the launch picks 8-wave workgroups
    g = torch.Generator(device=DEV).manual_seed(3000 + Sq + Skv + d)
    q = torch.randn((B, Hq, Sq, d), generator=g, device=DEV).to(torch.bfloat16)
    k = torch.randn((B, Hkv, Skv, d), generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn((B, Hkv, Skv, d), generator=g, device=DEV).to(torch.bfloat16)
    scale = 1.0 / math.sqrt(d)
    o, lse = nan_outputs(q)
    sa.prefill(q, k, v, causal=causal, scale=scale, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all(), "an output row was not written"
    rows = sorted(r for r in set(block_rows(Sq, np.random.default_rng(Sq + Skv), block=32)) | {1, 127, 128, 255, 256}
                  if r < Sq)
    check_prefill_rows(o, lse, q, k, v, scale, causal, rows)


# The 8-wave (two-team) launch over short key ranges: one to five 64-key
# tiles, fewer than the loop's three-slot rings hold, so the prologue, the
# second team's first half-step and the idle tail half-steps all run.  Every
# output element is checked.
EIGHT_WAVE_SHORT = [
    # B, Hq, Hkv, Sq, Skv, d, causal
    (16, 64, 8, 64, 64, 128, True),       # one tile
    (16, 64, 8, 64, 128, 128, False),     # two tiles
    (16, 64, 8, 100, 150, 128, True),     # three tiles, ragged last tile and query block
    (16, 64, 8, 64, 250, 64, False),      # four tiles, d = 64
    (16, 64, 8, 40, 300, 128, True),      # five tiles, each wave ending at a different tile
]


@pytest.mark.parametrize("B,Hq,Hkv,Sq,Skv,d,causal", EIGHT_WAVE_SHORT)
def test_eight_wave_launch_short_key_ranges(B, Hq, Hkv, Sq, Skv, d, causal):
    assert -(-(Hq // Hkv) * Sq // 256) * B * Hkv >= 256 and (Hq // Hkv) * Sq > 128   # 8-wave workgroups
    assert sa.prefill_splits(B, Hq, Hkv, Sq, Skv) == 1
    g = torch.Generator(device=DEV).manual_seed(4000 + Sq + Skv + d)
    q = torch.randn((B, Hq, Sq, d), generator=g, device=DEV).to(torch.bfloat16)
    k = torch.randn((B, Hkv, Skv, d), generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn((B, Hkv, Skv, d), generator=g, device=DEV).to(torch.bfloat16)
    run_and_check(q, k, v, causal)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("step", [2.0, -1.0])
def test_eight_wave_scores_that_climb_or_fall_across_tiles(step, causal):
    """As the drift test above, in the 8-wave (two-team) launch: there the
    range guard's redo reads the tile's K back from its LDS slot while the
    other team runs, and the owed O rescale is applied in the next matrix
    phase."""
    B, Hq, Hkv, Sq, Skv, d = 16, 64, 8, 64, 600, 128
    assert -(-(Hq // Hkv) * Sq // 256) * B * Hkv >= 256 and sa.prefill_splits(B, Hq, Hkv, Sq, Skv) == 1
    g = torch.Generator(device=DEV).manual_seed(int(100 * step) + 7 + causal)
    q = (1.0 + 0.25 * torch.randn((B, Hq, Sq, d), generator=g, device=DEV)).to(torch.bfloat16)
    drift = step * (torch.arange(Skv, device=DEV) // 64).float()
    k = (drift[None, None, :, None] + 0.25 * torch.randn((B, Hkv, Skv, d), generator=g, device=DEV)).to(torch.bfloat16)
    v = torch.randn((B, Hkv, Skv, d), generator=g, device=DEV).to(torch.bfloat16)
    o, lse = run_and_check(q, k, v, causal)
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()


def test_lse_output_is_optional():
    """lse = NULL writes O only, bitwise the same O as with the LSE output (both
    launch shapes: 4-wave small, 8-wave large)."""
    for (Hq, Hkv, S) in ((8, 2, 300), (64, 8, 2048)):
        g = torch.Generator(device=DEV).manual_seed(4000 + S)
        q = torch.randn((1, Hq, S, 128), generator=g, device=DEV).to(torch.bfloat16)
        k = torch.randn((1, Hkv, S, 128), generator=g, device=DEV).to(torch.bfloat16)
        v = torch.randn((1, Hkv, S, 128), generator=g, device=DEV).to(torch.bfloat16)
        o1, _ = sa.prefill(q, k, v, causal=True)
        o2 = sa.prefill(q, k, v, causal=True, return_lse=False)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2)

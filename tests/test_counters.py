"""Recorded hardware counters against what the kernels' schedules imply
(host arithmetic only; the counts come from rocprofv3 runs summarised under
profiles/)."""

# SQ_INSTS_MFMA of one 70B-shape causal prefill launch (B=1, 64/8 heads,
# S=8192, d=128; two-team kernel), profiles/prefill_lds_mfma_counters_70b.md.
MEASURED_PREFILL_MFMA = 33_816_576
# FETCH_SIZE and WRITE_SIZE (KiB per launch) of the same launch, and the
# copy calibration (FETCH_SIZE reads half the bytes a plain copy moves,
# WRITE_SIZE all of them), profiles/hbm_traffic_70b_prefill_decode_chunked_paged.md.
MEASURED_PREFILL_FETCH_KIB = 137_339
MEASURED_PREFILL_WRITE_KIB = 133_120
FETCH_SCALE, WRITE_SCALE = 0.5, 1.0
# FETCH_SIZE (KiB) of the decode split kernel and the KV bytes it must read.
MEASURED_DECODE_FETCH_KIB = 262_253
DECODE_KV_BYTES = 4 * 8 * 32768 * 128 * 2 * 2
# FETCH_SIZE (KiB) of the paged decode kernel (16 sequences x 4 tokens, 64/8
# heads, lengths summing to 286,824 keys, 64-position pages shuffled in the
# pool), the K/V bytes of the valid keys and the Q bytes.
MEASURED_PAGED_FETCH_KIB = 574_406
PAGED_KV_BYTES = 286_824 * 8 * 128 * 2 * 2
PAGED_Q_BYTES = 16 * 64 * 4 * 128 * 2

PREFILL_B, PREFILL_HQ, PREFILL_HKV, PREFILL_S, PREFILL_D = 1, 64, 8, 8192, 128


def prefill_mfma_count(S, G, Hkv, rows_per_wave=32, key_tile=64, d=128):
    """MFMA instructions of a causal prefill (Sq = Skv = S) in the two-team
    kernel.  A wave holds 32 positions of one query head (with G = 8 a
    workgroup is the same 32 positions of the 8 heads) and computes, for
    every key tile it sees, that tile's scores (the first in the prologue,
    the others in the matrix phase before) and its P V product: the score
    MFMAs of the tile after its last one are not issued."""
    per_tile = 2 * (d // 16)          # 32x32x16 MFMAs for 64 keys x 32 rows (scores), and as many for P V
    total = 0
    for _ in range(Hkv * G):
        for t0 in range(0, S, rows_per_wave):
            tiles = -(-(t0 + rows_per_wave) // key_tile)   # causal: keys up to the wave's last row
            total += 2 * per_tile * tiles
    return total


def prefill_algorithmic_bytes():
    """Q, K, V read once; O (bf16) and LSE (fp32) written once."""
    q = PREFILL_B * PREFILL_HQ * PREFILL_S * PREFILL_D * 2
    kv = 2 * PREFILL_B * PREFILL_HKV * PREFILL_S * PREFILL_D * 2
    o = q
    lse = PREFILL_B * PREFILL_HQ * PREFILL_S * 4
    return q, kv, o + lse


def test_prefill_issues_exactly_the_mfmas_of_its_causal_schedule():
    assert prefill_mfma_count(PREFILL_S, PREFILL_HQ // PREFILL_HKV, PREFILL_HKV) == MEASURED_PREFILL_MFMA


def test_prefill_hbm_traffic_stays_within_one_and_a_half_times_the_minimum():
    q, kv, out = prefill_algorithmic_bytes()
    fetched = MEASURED_PREFILL_FETCH_KIB * 1024 / FETCH_SCALE
    written = MEASURED_PREFILL_WRITE_KIB * 1024 / WRITE_SCALE
    assert fetched >= q + kv and written >= out                      # nothing is read or written less than once
    assert fetched + written <= 1.5 * (q + kv + out)
    assert written <= 1.01 * out                                    # O and LSE written once


def test_prefill_kv_reads_share_the_group():
    """The G = 8 query heads of a KV head read its K/V tiles together (one
    workgroup holds the same 32 positions of all 8 heads), so the K/V bytes
    fetched from memory stay far below one fetch per query head."""
    q, kv, _ = prefill_algorithmic_bytes()
    kv_fetched = MEASURED_PREFILL_FETCH_KIB * 1024 / FETCH_SCALE - q
    G = PREFILL_HQ // PREFILL_HKV
    assert kv_fetched <= 5 * kv < G * kv


def test_decode_fetches_each_kv_byte_once():
    fetched = MEASURED_DECODE_FETCH_KIB * 1024 / FETCH_SCALE
    assert DECODE_KV_BYTES <= fetched <= 1.002 * DECODE_KV_BYTES


def test_paged_decode_fetches_each_valid_kv_byte_once():
    """Pages are read only up to each sequence's length (rows past it in the
    last page are never fetched) and each valid K/V byte once."""
    fetched = MEASURED_PAGED_FETCH_KIB * 1024 / FETCH_SCALE
    assert PAGED_KV_BYTES <= fetched <= 1.002 * (PAGED_KV_BYTES + PAGED_Q_BYTES)

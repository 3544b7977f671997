"""Recorded hardware counters against what the kernels' schedules imply
(host arithmetic only; the counts come from rocprofv3 runs summarised under
profiles/)."""

# SQ_INSTS_MFMA of one 70B-shape causal prefill launch (B=1, 64/8 heads,
# S=8192, d=128), profiles/prefill_lds_mfma_counters_70b.md.
MEASURED_PREFILL_MFMA = 34_537_472
# FETCH_SIZE (KiB, copy-calibrated x2) of the decode split kernel and the KV
# bytes it must read, profiles/hbm_traffic_70b_prefill_decode_chunked_paged.md.
MEASURED_DECODE_FETCH_KIB = 262_469
DECODE_KV_BYTES = 4 * 8 * 32768 * 128 * 2 * 2


def prefill_mfma_count(S, G, Hkv, rows_per_wg=256, waves=8, key_tile=64, d=128):
    """MFMA instructions of a causal prefill (Sq = Skv = S): per wave, the
    first tile's scores, then one step per key tile up to the wave's last
    visible tile (score MFMAs of the next tile + P V MFMAs of the previous
    one), then the last tile's P V product if the wave reaches it."""
    per_tile = 2 * (d // 16)          # 32x32x16 MFMAs for 64 keys x 32 rows (scores), and as many for P V
    total = 0
    for _ in range(Hkv * G):
        for t0 in range(0, S, rows_per_wg):
            kt_hi = -(-(t0 + rows_per_wg) // key_tile)
            for w in range(waves):
                rows = rows_per_wg // waves
                wave_end = min(-(-(t0 + rows * (w + 1)) // key_tile), kt_hi)
                steps = min(wave_end, kt_hi - 1) + 1
                total += per_tile + 2 * per_tile * steps + (per_tile if wave_end >= kt_hi else 0)
    return total


def test_prefill_issues_exactly_the_mfmas_of_its_causal_schedule():
    assert prefill_mfma_count(8192, 8, 8) == MEASURED_PREFILL_MFMA


def test_decode_fetches_each_kv_byte_once():
    fetched = MEASURED_DECODE_FETCH_KIB * 1024 * 2          # FETCH_SIZE counts half the bytes (copy calibration)
    assert DECODE_KV_BYTES <= fetched <= 1.002 * DECODE_KV_BYTES

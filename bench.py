#!/usr/bin/env python3
"""Benchmark of the streaming attention hot path on one MI355X.

One step = one pass of the whole path on resident synthetic inputs:
  * causal GQA prefill, Llama3-70B head shape: B=1, 64 query / 8 KV heads,
    S=8192, d=128, bf16 (attn_prefill), and
  * split-KV GQA decode: B=4, 64/8 heads, KV cache 32768 tokens, d=128, bf16,
    64 splits per sequence (attn_decode_splitkv + attn_combine_lse).

Prints ONE JSON line.  `value` is the prefill throughput in algorithmic TFLOP/s
(4 * d * visible (q, k) pairs per head / prefill kernel time); the decode
throughput in KV GB/s (every valid K and V byte once / split + combine time)
is reported next to it.  Outside the step, after it, these are timed on their
own and reported under their own keys:
  * `ragged_decode`: split-KV decode of 16 sequences with lengths uniform in
    [1024, 131072], split count per length, + merge;
  * `chunked_prefill`: 512 queries after a 65536-token prefix, split-KV + merge;
  * `mha_causal_prefill`: causal MHA prefill B=2, H=16, S=1024, d=64 (report
    only: a launch-latency-sized problem);
  * `paged_decode`: multi-token decode over a paged cache (16 sequences x 4
    tokens, lengths 1K-32K).
Kernel times come from HIP events recorded on the stream the kernels run on,
over the timed steps; the events are created with hipEventDisableSystemFence
(timing only, no system-scope cache writeback at each record, see Timer).  The float64 oracle, timed on
the host cores on a bounded sample of the same prefill workload, is reported as
`cpu_baseline` (a baseline only).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Defaults: 20 warmup steps, 30 timed.  The GPU's clock settles only after some
tens of milliseconds of this load: in a kernel trace the prefill's first
launches take up to 1.2 ms and later ones 0.98 ms.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 flop/clk (dense bf16)
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
METRIC = "prefill TFLOP/s (%MFMA peak); decode KV GB/s (%HBM peak), 70B-shape GQA"

# Measured HBM bytes per launch of the dominant kernels: two rocprofv3 --pmc runs
# (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch) on `bench.py --only prefill|decode|chunked|paged`,
# each scaled by what the same counter reads for a plain 1 GiB device copy
# (`bench.py --only copy`: FETCH_SIZE reads 0.5x the copied bytes, WRITE_SIZE 1.0x).
# Each entry holds for the kernel sources whose hash it records; after any change to
# them the bench reports traffic as null until the counters are taken again.
# Summary and commands: profiles/hbm_traffic_70b_prefill_decode_chunked_paged.md.
FETCH_SCALE = 0.5
WRITE_SCALE = 1.0
TRAFFIC = {
    "prefill": {"sources": ["common.h", "prefill.hip"], "sha256_16": "ddc01e2fae5a9f54",
                "fetch_kib": 137339, "write_kib": 133120},
    "decode": {"sources": ["common.h", "decode.hip", "combine.hip"], "sha256_16": "05ddfcb1dded8f23",
               "fetch_kib": 262253 + 4170, "write_kib": 8256 + 65},
    "chunked": {"sources": ["common.h", "prefill.hip", "combine.hip"], "sha256_16": "4739eee8bdee01c4",
                "fetch_kib": 140440 + 16914, "write_kib": 33280 + 8448},
    "paged": {"sources": ["common.h", "paged.hip", "combine.hip"], "sha256_16": "f2459d9c52b18dfe",
              "fetch_kib": 574406 + 6258, "write_kib": 12391 + 1056},
    "ragged": {"sources": ["common.h", "decode.hip", "combine.hip"], "sha256_16": "05ddfcb1dded8f23",
               "fetch_kib": 2031568 + 8203, "write_kib": 16268 + 260},
}


def code_hash(sources):
    """First 16 hex digits of the SHA-256 of the kernel sources' code: each
    file with its // comments, trailing blanks and empty lines removed, so that
    a comment edit does not retire the counters."""
    import hashlib
    import re
    m = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, "streaming_attention_amd", "csrc", f), encoding="utf-8") as fh:
            text = re.sub(r"//[^\n]*", "", fh.read())
        m.update("\n".join(ln.rstrip() for ln in text.splitlines() if ln.strip()).encode())
    return m.hexdigest()[:16]


def measured_traffic(name):
    """HBM bytes per launch (fetch + write, copy-calibrated), or None if stale."""
    t = TRAFFIC[name]
    if t["sha256_16"] is None or code_hash(t["sources"]) != t["sha256_16"]:
        return None
    return int(t["fetch_kib"] * 1024 / FETCH_SCALE + t["write_kib"] * 1024 / WRITE_SCALE)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["all", "prefill", "decode", "chunked", "paged", "ragged", "mha", "copy"],
                    default="all",
                    help="run only one part (for per-kernel profiling runs): one half of the step, the "
                         "chunked prefill, the paged multi-token decode, the ragged decode, the small MHA "
                         "prefill, or 'copy', a plain 1 GiB device copy that is the reference for scaling "
                         "HBM byte counters")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target wall time of the oracle sample")
    return ap.parse_args()


def cpu_baseline(target_s: float):
    """Time the float64 oracle on whole query heads of the prefill workload
    (all 8192 rows of head 0, 1, ... until about target_s seconds)."""
    import oracle
    from streaming_attention_amd import workloads as W

    w = W.GQA70B_PREFILL
    q, k, v = W.prefill_inputs(w, "cpu")          # the same seeded inputs as the GPU leg
    G = w.Hq // w.Hkv
    heads = 0
    el = 0.0
    kv_np = {}
    while heads < w.Hq:
        kvh = heads // G
        if kvh not in kv_np:
            kv_np = {kvh: (k[:, kvh:kvh + 1].float().numpy(), v[:, kvh:kvh + 1].float().numpy())}
        kh, vh = kv_np[kvh]
        qh = q[:, heads:heads + 1].float().numpy()
        t0 = time.perf_counter()
        oracle.attention(qh, kh, vh, w.scale, True)
        el += time.perf_counter() - t0
        heads += 1
        if el >= target_s:
            break
    flops = 4 * w.d * w.visible_pairs_per_head() * heads
    threads = os.cpu_count()
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        if info:
            threads = max(int(i.get("num_threads", 0)) for i in info) or threads
    except Exception:
        pass
    return {
        "value": round(flops / el / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"float64 oracle (score matrix materialised per head) on {heads} of the {w.Hq} query heads "
                  f"(all {w.Sq} rows each) of the causal S={w.Skv} d={w.d} GQA prefill; {el:.1f} s of oracle time; "
                  f"value = algorithmic flops of those heads / that time",
    }


class Timer:
    """Timing events on the launch stream.

    The events are HIP events created with hipEventDisableSystemFence, on the
    HIP runtime the process already has loaded (the one torch uses).  A
    default event's recording releases at system scope, which writes back and
    invalidates the GPU caches; the kernel that follows then starts late and
    on cold caches, and that cost lands in the next timing window (measured:
    +2 to 3 us on the 93 us decode after the prefill).  HIP documents the flag
    for exactly this use: events that only time work.  If the runtime cannot
    be found, torch's default events are used and the JSON says so."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, stream):
        import ctypes
        import re

        import torch

        self.stream = stream
        self.hip = None
        try:
            maps = open("/proc/self/maps", encoding="utf-8").read()
            paths = sorted(set(re.findall(r"(/\S*libamdhip64\S*)", maps)))
            if paths:
                hip = ctypes.CDLL(paths[0], mode=os.RTLD_NOLOAD | os.RTLD_GLOBAL)
                for name in ("hipEventCreateWithFlags", "hipEventRecord", "hipEventSynchronize",
                             "hipEventElapsedTime", "hipEventDestroy"):
                    getattr(hip, name).restype = ctypes.c_int
                self.hip = hip
        except OSError:
            self.hip = None
        self._ctypes = ctypes
        self._torch = torch
        self._live = []
        self.kind = ("HIP events with hipEventDisableSystemFence on the launch stream" if self.hip is not None
                     else "torch.cuda.Event on the launch stream (HIP runtime not found)")

    def event(self):
        if self.hip is None:
            return self._torch.cuda.Event(enable_timing=True)
        e = self._ctypes.c_void_p()
        if self.hip.hipEventCreateWithFlags(self._ctypes.byref(e), self._ctypes.c_uint(self.DISABLE_SYSTEM_FENCE)):
            raise RuntimeError("hipEventCreateWithFlags failed")
        self._live.append(e)
        return e

    def record(self, e):
        if self.hip is None:
            e.record(self.stream)
        elif self.hip.hipEventRecord(e, self._ctypes.c_void_p(self.stream.cuda_stream)):
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b):
        if self.hip is None:
            return a.elapsed_time(b)
        if self.hip.hipEventSynchronize(b):
            raise RuntimeError("hipEventSynchronize failed")
        ms = self._ctypes.c_float()
        if self.hip.hipEventElapsedTime(self._ctypes.byref(ms), a, b):
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def close(self):
        if self.hip is not None:
            for e in self._live:
                self.hip.hipEventDestroy(e)
        self._live = []


def timed_mean_ms(fn, warmup: int, steps: int, timer: Timer) -> float:
    """Mean time of one call of fn over `steps` calls after `warmup` untimed
    ones: timing events recorded on the launch stream around the timed calls."""
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = timer.event(), timer.event()
    timer.record(e0)
    for _ in range(steps):
        fn()
    timer.record(e1)
    torch.cuda.synchronize()
    return timer.elapsed_ms(e0, e1) / steps


def measure_ragged(sa, W, dev, timer, warmup, steps):
    """Ragged decode: B=16, lengths uniform in [1024, 131072] from the seed,
    splits per length (splits_for_lengths), split-KV + merge."""
    import torch

    wr = W.RAGGED_DECODE
    qr, kr, vr, lens_r = W.decode_inputs(wr, dev)
    ns = sa.splits_for_lengths(lens_r)
    lens_d, ns_d = lens_r.to(dev), ns.to(dev)
    po = torch.empty((wr.B, wr.Hq, 64, wr.d), dtype=torch.float32, device=dev)
    pl = torch.empty((wr.B, wr.Hq, 64), dtype=torch.float32, device=dev)
    o = torch.empty((wr.B, wr.Hq, 1, wr.d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((wr.B, wr.Hq), dtype=torch.float32, device=dev)

    def call():
        sa.decode(qr, kr, vr, lens_d, ns_d, max_splits=64, scale=wr.scale, part_o=po, part_lse=pl, out=o, lse=lse)

    ms = timed_mean_ms(call, warmup, steps, timer)
    kv = W.decode_kv_bytes(lens_r, wr.Hkv, wr.d)
    gbs = kv / (ms * 1e-3) / 1e9
    return {"workload": f"ragged split-KV decode B={wr.B} Hq={wr.Hq} Hkv={wr.Hkv} d={wr.d} bf16, lengths "
                        f"U[{wr.len_lo},{wr.len_hi}] (seed {wr.seed}: sum {int(lens_r.sum())}), splits per "
                        f"length min(64, ceil(len/2048)) (sum {int(ns.sum())})",
            "kernels": "decode_splitkv_bf16_kernel<128> + combine_lse_kernel<128>",
            "us": round(ms * 1e3, 2), "kv_gbs": round(gbs, 1), "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
            "kv_bytes": kv,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic("ragged"),
                         "traffic_unit": "HBM bytes per call, split + merge (fetch + write)"}}


def measure_mha(sa, W, dev, timer, warmup, steps):
    """Causal MHA prefill B=2, H=16, S=1024, d=64 (bf16): report only."""
    import torch

    wm = W.MHA_CAUSAL
    qm, km, vm = W.prefill_inputs(wm, dev)
    om = torch.empty_like(qm)
    lsem = torch.empty((wm.B, wm.Hq, wm.Sq), dtype=torch.float32, device=dev)
    ms = timed_mean_ms(lambda: sa.prefill(qm, km, vm, causal=True, scale=wm.scale, out=om, lse=lsem),
                       warmup, steps, timer)
    tf = wm.flops() / (ms * 1e-3) / 1e12
    return {"workload": f"causal MHA prefill B={wm.B} H={wm.Hq} S={wm.Sq} d={wm.d} bf16 (report only)",
            "kernels": "prefill_bf16_kernel<64,causal>", "us": round(ms * 1e3, 2), "tflops": round(tf, 2),
            "pct_mfma_peak": round(100 * tf / MFMA_BF16_PEAK_TFLOPS, 2),
            "algorithmic_gflop": round(wm.flops() / 1e9, 4)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(no collectives or multi-GPU sharding in this library).", file=sys.stderr)
        sys.exit(2)

    import torch

    import streaming_attention_amd as sa
    from streaming_attention_amd import workloads as W

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.only == "copy":
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": args.warmup + args.steps}))
        return
    wp = W.GQA70B_PREFILL
    wd = W.GQA70B_DECODE

    q, k, v = W.prefill_inputs(wp, dev)
    o = torch.empty_like(q)
    lse = torch.empty((wp.B, wp.Hq, wp.Sq), dtype=torch.float32, device=dev)
    qd, kc, vc, lens = W.decode_inputs(wd, dev)
    part_o = torch.empty((wd.B, wd.Hq, wd.splits, wd.d), dtype=torch.float32, device=dev)
    part_lse = torch.empty((wd.B, wd.Hq, wd.splits), dtype=torch.float32, device=dev)
    od = torch.empty((wd.B, wd.Hq, 1, wd.d), dtype=torch.bfloat16, device=dev)
    lsed = torch.empty((wd.B, wd.Hq), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    timer = Timer(stream)
    n_ev = args.steps
    ev = [[timer.event() for _ in range(3)] for _ in range(n_ev)]

    do_pf = args.only in ("all", "prefill")
    do_dc = args.only in ("all", "decode")
    do_ch = args.only in ("all", "chunked")
    do_pg = args.only in ("all", "paged")
    do_rg = args.only in ("all", "ragged")
    do_mh = args.only in ("all", "mha")

    def step(i=None):
        if i is not None:
            timer.record(ev[i][0])
        if do_pf:
            sa.prefill(q, k, v, causal=True, scale=wp.scale, out=o, lse=lse)
        if i is not None:
            timer.record(ev[i][1])
        if do_dc:
            sa.decode(qd, kc, vc, None, None, max_splits=wd.splits, scale=wd.scale,
                      part_o=part_o, part_lse=part_lse, out=od, lse=lsed)
        if i is not None:
            timer.record(ev[i][2])

    wall = 0.0
    if do_pf or do_dc:
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(i)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0

    pf_ms = dc_ms = float("nan")
    if do_pf or do_dc:
        pf_ms = sum(timer.elapsed_ms(ev[i][0], ev[i][1]) for i in range(n_ev)) / n_ev
        dc_ms = sum(timer.elapsed_ms(ev[i][1], ev[i][2]) for i in range(n_ev)) / n_ev
    ms_step = wall * 1e3 / args.steps

    ragged = None
    if do_rg:   # ragged split-KV decode + merge, timed on its own (not part of the step)
        ragged = measure_ragged(sa, W, dev, timer, args.warmup, args.steps)
        torch.cuda.empty_cache()

    mha = None
    if do_mh:
        mha = measure_mha(sa, W, dev, timer, args.warmup, args.steps)

    chunked = None
    if do_ch:   # split-KV prefill + merge, timed on its own (not part of the step)
        wc = W.CHUNKED_PREFILL
        qc, kc2, vc2 = W.prefill_inputs(wc, dev)
        oc = torch.empty_like(qc)
        lsec = torch.empty((wc.B, wc.Hq, wc.Sq), dtype=torch.float32, device=dev)
        n_sp = sa.prefill_splits(wc.B, wc.Hq, wc.Hkv, wc.Sq, wc.Skv)
        ch_ms = timed_mean_ms(lambda: sa.prefill(qc, kc2, vc2, causal=True, scale=wc.scale, out=oc, lse=lsec),
                              args.warmup, args.steps, timer)
        ch_tf = wc.flops() / (ch_ms * 1e-3) / 1e12
        chunked = {"workload": f"causal chunked prefill B={wc.B} Hq={wc.Hq} Hkv={wc.Hkv} Sq={wc.Sq} "
                               f"Skv={wc.Skv} (query block after a {wc.Skv - wc.Sq}-token prefix) d={wc.d} bf16",
                   "kv_splits": n_sp, "kernels": "prefill_pp_kernel<128,causal> (split-KV, two-team) + combine_lse",
                   "ms": round(ch_ms, 4), "tflops": round(ch_tf, 2),
                   "pct_mfma_peak": round(100 * ch_tf / MFMA_BF16_PEAK_TFLOPS, 2),
                   "algorithmic_tflop": round(wc.flops() / 1e12, 6),
                   "traffic": measured_traffic("chunked"),
                   "traffic_unit": "HBM bytes per call, split-KV prefill + merge (fetch + write)"}
        del qc, kc2, vc2, oc, lsec

    paged = None
    if do_pg:   # multi-token decode over a paged cache, timed on its own (not part of the step)
        wg = W.PAGED_DECODE
        qg, kpg, vpg, tbl, lens_g = W.paged_inputs(wg, dev)
        tbl_d, lens_d = tbl.to(dev), lens_g.to(dev)
        og = torch.empty((wg.B, wg.Hq, wg.T_q, wg.d), dtype=torch.bfloat16, device=dev)
        lseg = torch.empty((wg.B, wg.Hq, wg.T_q), dtype=torch.float32, device=dev)
        n_sp = sa.paged_splits(wg.B, wg.Hq, wg.Hkv, wg.T_q, tbl.shape[1])
        pg_ms = timed_mean_ms(lambda: sa.decode_paged(qg, kpg, vpg, tbl_d, lens_d, scale=wg.scale, out=og, lse=lseg),
                              args.warmup, args.steps, timer)
        pg_bytes = W.decode_kv_bytes(lens_g, wg.Hkv, wg.d)
        pg_gbs = pg_bytes / (pg_ms * 1e-3) / 1e9
        paged = {"workload": f"multi-token decode over a paged cache: B={wg.B} T_q={wg.T_q} Hq={wg.Hq} Hkv={wg.Hkv} "
                             f"d={wg.d} bf16, lengths U[{wg.len_lo},{wg.len_hi}] (sum {int(lens_g.sum())}), "
                             f"pages of {wg.page} shuffled in the pool",
                 "kv_splits": n_sp,
                 "kernels": "decode_paged_bf16_kernel<128> (split-KV) + combine_lse",
                 "us": round(pg_ms * 1e3, 2), "kv_gbs": round(pg_gbs, 1),
                 "pct_hbm_peak": round(100 * pg_gbs / HBM_PEAK_GBS, 2), "kv_bytes": pg_bytes,
                 "traffic": measured_traffic("paged"),
                 "traffic_unit": "HBM bytes per call, paged split-KV + merge (fetch + write)"}
        del qg, kpg, vpg, tbl_d, lens_d, og, lseg

    pf_flops = wp.flops()
    pf_tflops = pf_flops / (pf_ms * 1e-3) / 1e12 if do_pf else 0.0
    kv_bytes = W.decode_kv_bytes(lens, wd.Hkv, wd.d)
    dc_gbs = kv_bytes / (dc_ms * 1e-3) / 1e9 if do_dc else 0.0

    result = {
        "metric": METRIC,
        "value": round(pf_tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "70B-shape GQA step: causal prefill B=1 Hq=64 Hkv=8 S=8192 d=128 bf16 "
                        "+ split-KV decode B=4 Hq=64 Hkv=8 KV=32768 d=128 bf16, 64 splits",
            "prefill": {"B": wp.B, "Hq": wp.Hq, "Hkv": wp.Hkv, "Sq": wp.Sq, "Skv": wp.Skv, "d": wp.d,
                        "causal": True, "algorithmic_tflop": round(pf_flops / 1e12, 6)},
            "decode": {"B": wd.B, "Hq": wd.Hq, "Hkv": wd.Hkv, "kv_len": wd.fixed_len, "d": wd.d,
                       "splits": wd.splits, "kv_bytes": kv_bytes},
        },
        "prefill": {"ms": round(pf_ms, 4), "tflops": round(pf_tflops, 2),
                    "pct_mfma_peak": round(100 * pf_tflops / MFMA_BF16_PEAK_TFLOPS, 2)},
        "decode": {"us": round(dc_ms * 1e3, 2), "kv_gbs": round(dc_gbs, 1),
                   "pct_hbm_peak": round(100 * dc_gbs / HBM_PEAK_GBS, 2)},
        "roofline": {
            "bound": "mfma",
            "kernel": "prefill_pp_kernel<128,causal> (two-team, 8-wave workgroups)",
            "achieved": round(pf_tflops, 3),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(pf_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": measured_traffic("prefill"),
            "traffic_unit": "HBM bytes per launch (fetch + write)",
            "algorithmic_min_bytes": 2 * (2 * wp.B * wp.Hq * wp.Sq * wp.d + 2 * wp.B * wp.Hkv * wp.Skv * wp.d)
                                     + 4 * wp.B * wp.Hq * wp.Sq,
        },
        "roofline_decode": {
            "bound": "hbm",
            "kernel": "decode_splitkv_bf16_kernel<128> + combine_lse_kernel<128>",
            "achieved": round(dc_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(dc_gbs / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic("decode"),
            "traffic_unit": "HBM bytes per step, split + combine (fetch + write)",
            "algorithmic_bytes": kv_bytes,
        },
        "device": torch.cuda.get_device_name(dev),
        "timer": timer.kind,
    }
    if ragged is not None:
        result["ragged_decode"] = ragged
    if chunked is not None:
        result["chunked_prefill"] = chunked
    if mha is not None:
        result["mha_causal_prefill"] = mha
    if paged is not None:
        result["paged_decode"] = paged
    if not args.no_cpu_baseline:
        torch.cuda.empty_cache()
        result["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    timer.close()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

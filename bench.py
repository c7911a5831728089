#!/usr/bin/env python3
"""Benchmark of paged verify attention on one MI355X; prints ONE JSON line.

Default workload: one sequence, past_len 32768, 32 q heads / 8 KV heads
(GQA 4), head_dim 128, block 16, fp16 Q/KV/out, random block permutation —
a "step" is one pa_verify_forward call with T=3 verify rows (segment kernel +
combine kernel).  The same call with T=1 is timed beside it for the T-cost
ratio.  Inputs are resident in HBM before timing; KV pools are rotated over
>= 1 GiB of copies so the 256 MB Infinity Cache cannot serve them.

value = algorithmic KV bytes of one call / device time per call (GB/s), the
calls replayed from a HIP graph so host launch overhead is excluded (the
eager per-call time is reported beside it).
roofline = the segment kernel's algorithmic KV bytes / its own average
duration from HIP events its dispatch stamps (every 4th call of an eager
timed loop that keeps the GPU busy), against MI355X's 8 TB/s HBM peak.  cpu_baseline = the fp64 oracle timed on the host
cores over a bounded sample of the same call.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

HBM_PEAK_GBS = 8000.0
METRIC = "µs/call + achieved KV GB/s (% of HBM peak) at 32k ctx, T=3 vs T=1, 1 GPU"
ROTATE_BYTES = 1 << 30


def workloads():
    import pa_inputs as pi
    return {
        "gqa4_d128_f16_L32768": lambda T: pi.config2(32768, T),
        "gqa4_d128_f16_L8192": lambda T: pi.config2(8192, T),
        "gqa4_d128_f16_L32768_tree": lambda T: pi.config2(32768, T, tree=True),
        # the same cache in row-major pages ([num_blocks, Hkv, block_size, D])
        "gqa4_d128_f16_L32768_rowmajor": lambda T: pi.with_layout(pi.config2(32768, T), 1),
        "u8kv_d256_L32768_rowmajor": lambda T: pi.with_layout(pi.config3(32768, T), 1),
        "swa_pair_global_L32768_rowmajor": lambda T: pi.with_layout(pi.config4(32768, window=0, T=T), 1),
        "ragged8_bf16_rowmajor": lambda T: pi.with_layout(pi.config5(), 1),
        "gqa4_d128_f16_L32768_bs1": lambda T: pi.config2(32768, T, block_size=1),
        "gqa4_d128_f16_L32768_bs2": lambda T: pi.config2(32768, T, block_size=2),
        "gqa4_d128_f16_L32768_bs4": lambda T: pi.config2(32768, T, block_size=4),
        "gqa4_d128_f16_L32768_bs8": lambda T: pi.config2(32768, T, block_size=8),
        "u8kv_d256_L32768": lambda T: pi.config3(32768, T),
        # the same cache shapes at the other head sizes (not among the pages' workloads)
        "gqa4_d64_f16_L32768": lambda T: pi.build_case(
            [20, 32768, T], [32768], [T], num_q_heads=32, num_kv_heads=8, head_dim=64,
            block_size=16, name=f"gqa4_d64_f16_L32768_T{T}"),
        "u8kv_d64_L32768": lambda T: pi.build_case(
            [22, 32768, T], [32768], [T], num_q_heads=32, num_kv_heads=8, head_dim=64,
            block_size=16, kv_dtype=pi.U8, name=f"u8kv_d64_L32768_T{T}"),
        "u8kv_d128_L32768": lambda T: pi.build_case(
            [21, 32768, T], [32768], [T], num_q_heads=16, num_kv_heads=4, head_dim=128,
            block_size=16, kv_dtype=pi.U8, name=f"u8kv_d128_L32768_T{T}"),
        "swa_pair_global_L32768": lambda T: pi.config4(32768, window=0, T=T),
        "swa_pair_global_L51200": lambda T: pi.config4(51200, window=0, T=T),
        "swa_pair_window1024_L32768": lambda T: pi.config4(32768, window=1024, T=T),
        "ragged8_bf16": lambda T: pi.config5(),
        # batches of many sequences (fixed per-sequence segments: more
        # sequences than workgroup slots per KV head): past_len log-uniform,
        # shorter as the batch grows, T uniform in 1..4, bf16, 32 q / 8 KV
        # heads, head_dim 128, 16-slot pages
        "batch64_bf16": lambda T: pi.config5(num_seqs=64, lo=256, hi=4096, spare_blocks=8),
        "batch512_bf16": lambda T: pi.config5(num_seqs=512, lo=64, hi=1024, spare_blocks=8),
        "batch4096_bf16": lambda T: pi.config5(num_seqs=4096, lo=16, hi=256, spare_blocks=8),
    }


def kernel_source_hash():
    d = os.path.join(ROOT, "speculative_decoding_verify_paged_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".h")):
            h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload, T):
    """HBM bytes per segment-kernel launch from committed rocprofv3 counter
    runs, if they were taken on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        rec = json.load(open(p)).get(f"{workload}_T{T}")
    except (ValueError, OSError):
        return None
    if not rec or rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


class Runner:
    """Device-resident inputs for one case with rotated KV pool copies."""

    def __init__(self, case, copies=None):
        import torch
        from gpu_util import to_device
        import speculative_decoding_verify_paged_amd as pav
        self.pav = pav
        self.case = case
        self.dev = to_device(case)
        pool_bytes = sum(self.dev[k].numel() * self.dev[k].element_size()
                         for k in ("k_cache", "v_cache", "k_scale_zp", "v_scale_zp") if k in self.dev)
        self.copies = copies or max(1, math.ceil(ROTATE_BYTES / pool_bytes))
        self.pools = [self.dev]
        for _ in range(self.copies - 1):
            d = dict(self.dev)
            for k in ("k_cache", "v_cache", "k_scale_zp", "v_scale_zp"):
                if k in d:
                    d[k] = d[k].clone()
            self.pools.append(d)
        self.out = torch.empty_like(self.dev["q"])
        self.stream = torch.cuda.current_stream()
        # arguments marshalled once per pool copy: the timed loops issue only
        # the C call, so eager launches keep pace with the GPU
        c = case
        self.prepared = []
        opts = dict(sliding_window=c.sliding_window, max_query_len=max(c.Ts),
                    tree_mask=self.dev.get("tree_mask"), page_layout=c.page_layout)
        for d in self.pools:
            if c.kv_dtype == 2:
                pc = pav.prepare_forward_u8(d["q"], d["k_cache"], d["v_cache"], d["k_scale_zp"],
                                            d["v_scale_zp"], d["block_tables"], d["past_lens"],
                                            d["subsequence_begins"], c.max_context_len, c.scale,
                                            self.out, **opts)
            else:
                pc = pav.prepare_forward(d["q"], d["k_cache"], d["v_cache"], d["block_tables"],
                                         d["past_lens"], d["subsequence_begins"], c.max_context_len,
                                         c.scale, self.out, **opts)
            self.prepared.append(pc)

    def call(self, i, prof=None, stream=None):
        st = self.stream.cuda_stream if stream is None else stream
        self.prepared[i % self.copies](stream=st, prof_events=prof)

    def time_graph(self, steps, warmup, repeats):
        """µs per call with the `steps` calls captured in one HIP graph and
        replayed: device time per call, host launch overhead excluded (a
        serving engine replays the verify forward from a graph).  Each timed
        replay is enqueued right behind untimed replays of a second graph of
        the same calls, at least ~100 calls of them, so the timed calls start
        on a busy GPU and the host has enqueued them before it idles.  A
        timed replay still carries a fixed cost of its own on the device
        (~7 us on MI355X: the timing events and the graph's start and end),
        ~0.35 us per call at steps = 20.  Median and all values over
        `repeats` replays."""
        import torch
        for i in range(warmup):
            self.call(i)
        torch.cuda.synchronize()
        # two instances of the same calls: the untimed one runs while the
        # timed one is enqueued
        g, g_lead = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        for gr in (g, g_lead):
            with torch.cuda.graph(gr):
                cs = torch.cuda.current_stream().cuda_stream
                for i in range(steps):
                    self.call(i, stream=cs)
        torch.cuda.synchronize()
        g.replay()                                      # untimed replay
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        per_call = []
        lead = -(-100 // steps)                         # untimed replays ahead of the timed one
        for r in range(repeats):
            torch.cuda.synchronize()
            for _ in range(lead):
                g_lead.replay()                         # untimed, keeps the GPU busy
            t0.record()
            g.replay()
            t1.record()
            torch.cuda.synchronize()
            per_call.append(t0.elapsed_time(t1) * 1000.0 / steps)
        del g, g_lead
        return statistics.median(per_call), per_call

    def time(self, steps, warmup, repeats, stamp_every=4):
        """Eager launches: median µs per call and the segment kernel's mean
        duration from events its own dispatch stamps, over `repeats` regions.
        Every `stamp_every`-th call carries the events: a dispatch with events
        costs the host ~25 µs, so stamping every call would leave the GPU
        idle between calls instead of running them back to back."""
        import torch
        for i in range(warmup):
            self.call(i)
        torch.cuda.synchronize()
        per_call, per_kernel = [], []
        stamped = list(range(stamp_every - 1, steps, stamp_every))
        evb = {i: torch.cuda.Event(enable_timing=True) for i in stamped}
        eve = {i: torch.cuda.Event(enable_timing=True) for i in stamped}
        for e in list(evb.values()) + list(eve.values()):
            e.record(self.stream)           # create the underlying hipEvent
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        for r in range(repeats):
            torch.cuda.synchronize()
            t0.record(self.stream)
            for i in range(steps):
                self.call(i, prof=(evb[i].cuda_event, eve[i].cuda_event) if i in evb else None)
            t1.record(self.stream)
            torch.cuda.synchronize()
            per_call.append(t0.elapsed_time(t1) * 1000.0 / steps)
            per_kernel.append(statistics.mean(evb[i].elapsed_time(eve[i]) * 1000.0 for i in stamped))
        return statistics.median(per_call), statistics.median(per_kernel), per_call


def time_append(case, steps, warmup, repeats):
    """µs per pa_kv_append(_u8) call writing the case's T new tokens (values
    drawn once, stored in the q dtype), graph-replayed like the forward (the
    timed replay right behind untimed ones)."""
    import numpy as np
    import torch
    import speculative_decoding_verify_paged_amd as pav
    from gpu_util import to_device
    dev = to_device(case)
    rng = np.random.default_rng(1)
    qt = dev["q"].dtype
    shape = (case.num_tokens, case.num_kv_heads, case.head_dim)
    k_new = torch.from_numpy(rng.standard_normal(shape, dtype=np.float32)).cuda().to(qt)
    v_new = torch.from_numpy(rng.standard_normal(shape, dtype=np.float32)).cuda().to(qt)

    def one(stream):
        if case.kv_dtype == 2:
            pav.pa_kv_append_u8(k_new, v_new, dev["k_cache"], dev["v_cache"], dev["k_scale_zp"],
                                dev["v_scale_zp"], dev["block_tables"], dev["past_lens"],
                                dev["subsequence_begins"], max_query_len=max(case.Ts), stream=stream,
                                page_layout=case.page_layout)
        else:
            pav.pa_kv_append(k_new, v_new, dev["k_cache"], dev["v_cache"], dev["block_tables"],
                             dev["past_lens"], dev["subsequence_begins"], max_query_len=max(case.Ts),
                             stream=stream, page_layout=case.page_layout)

    for _ in range(warmup):
        one(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    g, g_lead = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    for gr in (g, g_lead):
        with torch.cuda.graph(gr):
            cs = torch.cuda.current_stream().cuda_stream
            for _ in range(steps):
                one(cs)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    per = []
    lead = -(-100 // steps)
    for _ in range(repeats):
        torch.cuda.synchronize()
        for _ in range(lead):
            g_lead.replay()                             # untimed, keeps the GPU busy
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) * 1000.0 / steps)
    e = 1 if case.kv_dtype == 2 else 2
    written = case.num_tokens * case.num_kv_heads * (2 * case.head_dim * e + (8 if e == 1 else 0))
    return {"us_per_call": round(statistics.median(per), 3), "bytes_written": written,
            "what": f"{case.num_tokens} new tokens x {case.num_kv_heads} KV heads into the "
                    f"{'u8 (quantised)' if e == 1 else 'f16/bf16'} cache"}


def read_ceiling():
    """Best HBM streaming-read rate of a plain 16-byte-load kernel over 4 GiB
    (beyond the 256 MB Infinity Cache), GB/s.  Also runs one 1 GiB copy, the
    known-size kernel that calibrates rocprofv3's FETCH_SIZE / WRITE_SIZE."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "speculative_decoding_verify_paged_amd", "libpa_membench.so"))
    lib.pa_membench_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                     ctypes.c_int, ctypes.c_void_p]
    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.zeros(1 << 16, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream()
    best = 0.0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for grid in (4096, 8192, 16384, 32768):
        for rep in range(3):
            torch.cuda.synchronize()
            e0.record()
            rc = lib.pa_membench_read(buf.data_ptr(), nbytes, sink.data_ptr(), grid, st.cuda_stream)
            e1.record()
            torch.cuda.synchronize()
            assert rc == 0
            best = max(best, nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    lib.pa_membench_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                     ctypes.c_int, ctypes.c_void_p]
    half = 1 << 30
    rc = lib.pa_membench_copy(buf.data_ptr() + half, buf.data_ptr(), half, 4096, st.cuda_stream)
    torch.cuda.synchronize()
    assert rc == 0
    del buf
    return round(best, 1)


def cpu_baseline(case, seconds):
    import oracle
    orc = oracle.get()
    n = 0
    t0 = time.perf_counter()
    while True:
        orc.forward(case)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    per = el / n
    return {"value": round(case.kv_bytes() / per / 1e9, 4), "unit": "GB/s", "cores": orc.num_threads(),
            "kind": "oracle", "seconds_per_call": round(per, 4),
            "sample": f"{n} full oracle call(s) of the timed workload ({case.num_tokens * case.num_q_heads} "
                      f"rows x {case.kv_keys()} keys), {el:.1f} s wall"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200, help="timed calls per timed region")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--repeats", type=int, default=5, help="timed regions; the median is reported")
    ap.add_argument("--workload", default="gqa4_d128_f16_L32768", choices=sorted(workloads()))
    ap.add_argument("--T", type=int, default=3, help="verify rows per sequence of the timed call")
    ap.add_argument("--no-t1", action="store_true", help="skip the T=1 comparison call")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the HBM read-ceiling kernel")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    mk = workloads()[args.workload]

    case = mk(args.T)
    run = Runner(case)
    us, spread = run.time_graph(args.steps, args.warmup, args.repeats)
    us_eager, us_kernel, _ = run.time(args.steps, args.warmup, args.repeats)
    kv = case.kv_bytes()
    copies = run.copies
    del run

    t1 = None
    if not args.no_t1 and args.T != 1 and args.workload.startswith("gqa4"):
        case1 = workloads()[args.workload.replace("_tree", "")](1)   # causal T = 1, same pages
        run1 = Runner(case1)
        us1, _ = run1.time_graph(args.steps, args.warmup, args.repeats)
        _, us1_kernel, _ = run1.time(args.steps, args.warmup, args.repeats)
        t1 = {"us_per_call": round(us1, 3), "us_segment_kernel": round(us1_kernel, 3),
              "kv_gbs": round(case1.kv_bytes() / us1 / 1e3, 1)}
        del run1
    append = time_append(case, args.steps, args.warmup, args.repeats)
    ceiling = None if args.no_ceiling else read_ceiling()

    value = kv / us / 1e3                                  # bytes/µs -> GB/s
    achieved = kv / us_kernel / 1e3
    traffic = measured_traffic(args.workload, args.T)
    dtype = {0: "f16", 1: "bf16", 2: "u8"}[case.kv_dtype]
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us / 1000.0, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": f"{args.workload}_T{args.T}", "num_seqs": case.num_seqs,
                   "past_lens": case.past_lens.tolist()[:8], "T": case.Ts[:8],
                   "q_heads": case.num_q_heads, "kv_heads": case.num_kv_heads,
                   "head_dim": case.head_dim, "block_size": case.block_size,
                   "sliding_window": case.sliding_window, "kv_dtype": dtype,
                   "tree_verify": case.tree_mask is not None,
                   "kv_bytes_per_call": kv, "pool_copies": copies},
        "us_per_call": round(us, 3),
        "us_per_call_spread": [round(x, 3) for x in spread],
        "us_per_call_eager": round(us_eager, 3),
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "hbm_read_ceiling_gbs": ceiling,
        "roofline": {"bound": "hbm", "kernel": "pa_segment_fp" if case.kv_dtype != 2 else "pa_segment_u8",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "kernel_us": round(us_kernel, 3), "traffic": traffic},
    }
    line["kv_append"] = append
    if t1 is not None:
        line["T1"] = t1
        line["t_over_t1"] = round(us / t1["us_per_call"], 4)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of the exact-attention hot path on one MI355X.

One step is one pass of the whole path over synthetic inputs already resident
in HBM:

* prefill forward on the non-causal batch-4, 32-head, N=4096 bf16 workload at
  d=64 and at d=128 (``attn_prefill_fwd``), and
* single-query split-K decode over one sequence's 262144-position bf16 cache
  with 32 query / 8 KV heads, d=128 (``attn_decode_splitk`` then
  ``attn_merge_partials``).

``value`` is the step's prefill throughput in algorithmic TFLOP/s (4·d FLOPs
per visible query-key pair) by wall clock over K steps after W warm-up steps,
``torch.cuda.synchronize`` on both sides; the decode half is a wall-clocked
region of its own and is reported in algorithmic KV GB/s (every K and V byte
read once) beside it.

Beside the step, each in a region of its own (warm-up, K wall-clocked
iterations), run the other workloads of the path: the causal GQA prefill
(N=32768, 32 query / 8 KV heads, d=128), the ragged batched decode (64
sequences of 1024..32768 cached positions, 64 query / 8 KV heads, q x8), the
one-head causal N=512 fp16 prefill (launch-bound: timed for completeness), the
262144-position decode over 16-row pages, the packed append batch (16
sequences of 256..2048 new queries on 0..16384 cached positions) and the
decode over the same cache as rotated 4-bit rows (encoded by the library's
``attn_kv_quantize_q4``).

Per-kernel durations: after each region's wall-clocked pass, a second pass of
max(K, 20) iterations brackets every launch with HIP events recorded on the
stream the kernels run on (events around every launch add stream overhead, so
they stay out of the wall-clocked pass).  ``kernels`` lists each kernel's mean
and median launch time and its algorithmic rate against the published peak of
its bound (``frac``) and against the ceiling measured on the same GPU in the
same run (``frac_of_measured``: a bf16 MFMA loop and a streaming read of 1 GiB,
``include/attn_calibrate.h``).  ``roofline`` is the step's dominant kernel,
with its mean launch time, the figure rocprofv3's kernel statistics average.
Inputs of the short kernels alternate between two copies so no launch finds
the previous one's data in the last-level cache; the decode caches (1 GiB and
more) exceed it by themselves.

``cpu_baseline`` times the fp64 oracle (test infrastructure, untuned) on the
host cores: whole (batch, head) slices of the d=128 step workload until about
``--cpu-seconds`` have passed, reported in TFLOP/s; ``cpu_baseline.configs``
adds the one-head N=512 prefill, the 262144-position decode and the ragged
decode in full, and one head of the causal N=32768 prefill (its whole-config
time extrapolated and labelled so).

``--summarize DIR`` turns rocprofv3 output under DIR into the text summaries
kept under ``profiles/`` (no GPU is touched).

Prints exactly one JSON line on stdout.  Only one GPU is supported.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "prefill TFLOP/s and decode KV GB/s on 1 MI355X, each as % of roofline"
PEAK_MFMA_BF16_TFLOPS = 2500.0   # MI355X dense bf16 (and fp16) matrix peak
PEAK_HBM_GBS = 8000.0            # MI355X HBM3E peak
C1 = "prefill_causal_b1_h1_n512_d64_f16"
C2 = ["prefill_b4_h32_n4096_d64_bf16", "prefill_b4_h32_n4096_d128_bf16"]
C3 = "prefill_causal_gqa_b1_hq32_hkv8_n32768_d128_bf16"
C4 = "decode_b1_hq32_hkv8_d128_len262144_bf16"
C5 = "decode_ragged_b64_hq64_hkv8_d128_len1024to32768_q8_bf16"
APPEND = "append_causal_b16_hq32_hkv8_d128_q256to2048_past0to16384_bf16"
PAGE_SIZE = 16
MIN_EVENT_LAUNCHES = 20
CSRC = os.path.join(ROOT, "exact_attention_flashattention_amd", "csrc")
KERNEL_SOURCES = {
    "prefill_fwd_kernel": ["prefill_fwd.hip", "device_common.hpp"],
    "decode_splitk_kernel": ["decode_splitk.hip", "device_common.hpp"],
    "merge_partials_kernel": ["merge_partials.hip", "device_common.hpp"],
    "decode_q4_kernel": ["decode_q4.hip", "device_common.hpp"],
    "quantize_q4_kernel": ["quantize_q4.hip", "device_common.hpp"],
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
ONLY = ["all", "step", "prefill_d64", "prefill_d128", "decode", "prefill_causal_gqa", "decode_ragged", "prefill_small",
        "decode_paged", "append", "decode_q4", "decode_q4_paged"]

# Kernels as rocprofv3 names them (template arguments), per bench label; the
# labels key the committed traffic counters.
ROCPROF_NAMES = {
    "prefill_fwd_kernel<bf16,d64,noncausal>": ("prefill_fwd_kernel<attn::Bf16, 64, false, false>", "prefill_d64"),
    "prefill_fwd_kernel<bf16,d128,noncausal>": ("prefill_fwd_kernel<attn::Bf16, 128, false, false>", "prefill_d128"),
    "prefill_fwd_kernel<bf16,d128,causal>": ("prefill_fwd_kernel<attn::Bf16, 128, true, false>", "prefill_causal_gqa"),
    "prefill_fwd_kernel<f16,d64,causal>": ("prefill_fwd_kernel<attn::F16, 64, true, false>", "prefill_small"),
    "decode_splitk_kernel<bf16,d128>": ("decode_splitk_kernel<attn::Bf16, 128, false>", "decode"),
    "merge_partials_kernel<bf16,d128>": ("merge_partials_kernel<attn::Bf16, 128", "decode"),
    "decode_splitk_kernel<bf16,d128,ragged>": ("decode_splitk_kernel<attn::Bf16, 128, false>", "decode_ragged"),
    "merge_partials_kernel<bf16,d128,ragged>": ("merge_partials_kernel<attn::Bf16, 128", "decode_ragged"),
    "decode_splitk_kernel<bf16,d128,paged16>": ("decode_splitk_kernel<attn::Bf16, 128, true>", "decode_paged"),
    "prefill_fwd_kernel<bf16,d128,causal,varlen>": ("prefill_fwd_kernel<attn::Bf16, 128, true, true>", "append"),
    "decode_q4_kernel<bf16,d128,rotated>": ("decode_q4_kernel<attn::Bf16, 128, false>", "decode_q4"),
    "decode_q4_kernel<bf16,d128,rotated,paged16>": ("decode_q4_kernel<attn::Bf16, 128, true>", "decode_q4_paged"),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_sha(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(label: str, kernel: str):
    """HBM bytes per launch from committed rocprofv3 FETCH_SIZE/WRITE_SIZE counts,
    if they were taken on the current source of the kernel; else None."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh).get("kernels", {}).get(label)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha") != source_sha(kernel):
        return None
    return rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return int(max((p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"),
                       default=1))
    except Exception:  # pragma: no cover
        return 1


# ---- CPU baseline: the oracle, untuned --------------------------------------------------------

def cpu_baseline(torch, workloads, dev, c2_inputs, seconds: float) -> dict:
    """The fp64 oracle on the host cores.  The headline figure: whole (batch,
    head) slices of the d=128 step workload until ``seconds`` have passed.
    ``configs``: the one-head N=512 prefill, the 262144-position decode and the
    ragged decode in full, and one head of the causal N=32768 prefill."""
    import numpy as np
    import oracle

    def f64(t):
        return t.detach().float().cpu().double().numpy()

    w = workloads.WORKLOADS[C2[1]]
    q, k, v = c2_inputs
    g = w.hq // w.hkv
    done, flops, elapsed = 0, 0.0, 0.0
    per_head = 4.0 * w.d * w.n * w.n
    for b in range(w.batch):
        for h in range(w.hq):
            qh, kh, vh = f64(q[b, h]), f64(k[b, h // g]), f64(v[b, h // g])
            t0 = time.perf_counter()
            oracle.attention(qh[None, None], kh[None, None], vh[None, None], w.scale, w.causal)
            elapsed += time.perf_counter() - t0
            done += 1
            flops += per_head
            if elapsed >= seconds:
                break
        if elapsed >= seconds:
            break
    host = f"host {cpu_model()}, {os.cpu_count()} logical CPUs"
    line = {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": blas_threads(), "kind": "oracle",
            "sample": f"{done} of {w.batch * w.hq} (batch, head) slices of {w.name}, whole rows, fp64 numpy; "
                      f"{elapsed:.1f} s; {host}"}
    configs = []

    # c1 in full
    w1 = workloads.WORKLOADS[C1]
    q1, k1, v1 = (f64(t) for t in workloads.prefill_inputs(w1))
    t0 = time.perf_counter()
    oracle.attention(q1, k1, v1, w1.scale, True)
    s = time.perf_counter() - t0
    configs.append({"workload": w1.name, "seconds": s, "value": w1.flops() / s / 1e12, "unit": "TFLOP/s",
                    "sample": "whole output"})

    # c4 and c5 in full, per (sequence, KV head), the caches read from the device
    for name in (C4, C5):
        wd = workloads.WORKLOADS[name]
        qd, kc, vc, lens = workloads.decode_inputs(wd, device=dev)
        gq = wd.hq // wd.hkv
        qf = f64(qd)
        s = 0.0
        for b in range(wd.batch):
            L = int(lens[b])
            for kh in range(wd.hkv):
                K, V = f64(kc[b, kh, :L]), f64(vc[b, kh, :L])
                t0 = time.perf_counter()
                oracle.attention_rows(qf[b, kh * gq:(kh + 1) * gq], K, V, wd.scale)
                s += time.perf_counter() - t0
        total = int(lens.sum())
        del kc, vc
        configs.append({"workload": wd.name, "seconds": s, "value": wd.kv_bytes(total) / s / 1e9, "unit": "GB/s",
                        "sample": "whole output (device-to-host copies and fp64 widening excluded)"})

    # c3: one head of 32 (the other heads cost the same), whole config extrapolated
    w3 = workloads.WORKLOADS[C3]
    q3, k3, v3 = workloads.prefill_inputs(w3, device=dev)
    qh, kh, vh = f64(q3[0, 0]), f64(k3[0, 0]), f64(v3[0, 0])
    del q3, k3, v3
    t0 = time.perf_counter()
    oracle.attention(qh[None, None], kh[None, None], vh[None, None], w3.scale, True)
    s = time.perf_counter() - t0
    configs.append({"workload": w3.name, "seconds": s * w3.hq, "value": w3.flops() / (s * w3.hq) / 1e12,
                    "unit": "TFLOP/s", "sample": f"query head 0 of {w3.hq} timed ({s:.1f} s); whole-config time "
                                                 f"EXTRAPOLATED x{w3.hq}"})
    line["configs"] = configs
    return line


# ---- measured ceilings -----------------------------------------------------------------------

def measured_ceilings(torch, lib, check, stream, reps: int = 10) -> dict:
    """Sustained bf16 MFMA rate and HBM read rate on this GPU (median of timed calls)."""
    blocks, iters = 512, 4096                      # two workgroups per CU on 256 CUs
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    buf = torch.ones(1 << 28, dtype=torch.float32, device="cuda")   # 1 GiB, far beyond the caches
    scratch = torch.empty(4096, dtype=torch.uint8, device="cuda")
    read_blocks = (2048, 4096, 8192)
    sp = stream.cuda_stream

    def timed(launch):
        for _ in range(3):
            launch()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            launch()
            e1.record(stream)
            e1.synchronize()
            ts.append(e0.elapsed_time(e1))
        return sorted(ts)[len(ts) // 2]

    ms_mfma = timed(lambda: check("attn_calib_mfma_bf16", lib.attn_calib_mfma_bf16(out.data_ptr(), blocks, iters, sp)))
    nbytes = buf.numel() * 4
    ms_read = min(timed(lambda rb=rb: check("attn_calib_read", lib.attn_calib_read(buf.data_ptr(), nbytes,
                                                                                   scratch.data_ptr(), rb, sp)))
                  for rb in read_blocks)
    flops = blocks * 4 * iters * 4 * 32768
    return {"mfma_bf16_tflops": flops / (ms_mfma * 1e-3) / 1e12, "hbm_read_gbs": nbytes / (ms_read * 1e-3) / 1e9,
            "how": f"attn_calib_mfma_bf16 ({blocks} workgroups x {iters} rounds of 4 MFMA chains) and "
                   f"attn_calib_read (1 GiB, best of {'/'.join(map(str, read_blocks))} workgroups); "
                   f"median of {reps} timed calls each"}


# ---- regions ---------------------------------------------------------------------------------

class Region:
    """A timed region: ``launch(i, ev)`` enqueues iteration i's kernels; with an
    event list it records event j before kernel j and the last one after the
    final kernel.  ``kernels`` describes each kernel: (label, source, bound,
    algorithmic work per launch, workload, extra fields)."""

    def __init__(self, name, launch, kernels, check=None):
        self.name, self.launch, self.kernels, self.check = name, launch, kernels, check
        self.wall_s = 0.0
        self.warm_launches = 0
        self.ms = []  # per kernel: list of event-timed launch durations


def run_region(torch, stream, reg: Region, K: int, W: int, warm_s: float = 0.0) -> None:
    # Untimed warm-up: W launches, continued until warm_s seconds have passed.  The shader clock
    # follows the load with a lag of milliseconds: after an idle moment, or after a kernel of a
    # different power draw, a prefill launch took up to 1.35x its settled time, recovering over
    # some 30 launches (per-dispatch kernel trace, per-workgroup time stamps).
    t0, i = time.perf_counter(), 0
    while i < W or time.perf_counter() - t0 < warm_s:
        reg.launch(i, None)
        i += 1
        if i % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    reg.warm_launches = i
    t0 = time.perf_counter()
    for i in range(K):
        reg.launch(i, None)
    torch.cuda.synchronize()
    reg.wall_s = time.perf_counter() - t0
    n = max(K, MIN_EVENT_LAUNCHES)
    nk = len(reg.kernels)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nk + 1)] for _ in range(n)]
    for i in range(n):
        reg.launch(i, evs[i])
    torch.cuda.synchronize()
    reg.ms = [[evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(n)] for j in range(nk)]
    if reg.check is not None:
        reg.check()


def kernel_records(reg: Region, in_step: bool):
    out = []
    for (label, src, bound, work, workload, extra), ms in zip(reg.kernels, reg.ms):
        mean, med = statistics.fmean(ms), statistics.median(ms)
        if bound == "mfma":
            rate, unit, peak = work / (mean * 1e-3) / 1e12, "TFLOP/s", PEAK_MFMA_BF16_TFLOPS
        else:
            rate, unit, peak = work / (mean * 1e-3) / 1e9, "GB/s", PEAK_HBM_GBS
        rec = {"kernel": label, "workload": workload, "avg_ms": mean, "median_ms": med, "launches": len(ms),
               "bound": bound, "achieved": rate, "peak": peak, "unit": unit, "frac": rate / peak,
               "achieved_at_median": rate * mean / med, "traffic": measured_traffic(label, src),
               ("algorithmic_flops" if bound == "mfma" else "algorithmic_bytes"): work, "in_step": in_step,
               "region": reg.name}
        rec.update(extra)
        out.append(rec)
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=8.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the measured MFMA-loop and streaming-read ceilings")
    ap.add_argument("--region-warmup-s", type=float, default=0.2,
                    help="each region's untimed warm-up lasts at least W launches and at least this many seconds")
    ap.add_argument("--only", choices=ONLY, default="all", help="run only one region or kernel (profiler runs)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="instead of the bench, run plain device copies of this many MiB (counter calibration)")
    ap.add_argument("--summarize", metavar="DIR", help="summarise rocprofv3 output under DIR (no GPU) and exit")
    ap.add_argument("--write-traffic", metavar="DIR",
                    help="write profiles/traffic_counters.json from FETCH_SIZE / WRITE_SIZE runs under DIR (no GPU)")
    args = ap.parse_args()

    if args.summarize:
        return summarize(args.summarize)
    if args.write_traffic:
        return write_traffic(args.write_traffic)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU: this build has no multi-GPU path (asked for --gpus "
              f"{args.gpus}, WORLD_SIZE={world}).", file=sys.stderr)
        return 2

    import torch

    import exact_attention_flashattention_amd as A
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    A._lib.load()

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(max(1, args.steps)):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {args.copy_calibration_mib} MiB x {max(1, args.steps)}")
        return 0

    stream = torch.cuda.current_stream(dev)
    K, W = args.steps, args.warmup
    only = args.only

    def want(*names):
        return only == "all" or only in names

    def mark(ev, j):
        if ev is not None:
            ev[j].record(stream)

    def partials(w, S, B=None):
        B = w.batch if B is None else B
        return (torch.empty((B, w.hq, S), dtype=torch.float32, device=dev),
                torch.empty((B, w.hq, S), dtype=torch.float32, device=dev),
                torch.empty((B, w.hq, S, w.d), dtype=torch.float32, device=dev))

    def finite(t, what):
        def f():
            if not torch.isfinite(t).all():
                raise RuntimeError(f"non-finite output on {what}")
        return f

    # ---- the step: prefill (N=4096, d=64 and d=128) + decode (L=262144)
    step_regions, other_regions = [], []
    c2_inputs = None
    for name in C2:
        d = workloads.WORKLOADS[name].d
        if not want("step", f"prefill_d{d}"):
            continue
        w = workloads.WORKLOADS[name]
        copies = [workloads.prefill_inputs(w, device=dev, salt=s) for s in (0, 1)]
        outs = [torch.empty_like(c[0]) for c in copies]
        if d == 128:
            c2_inputs = copies[0]

        def launch(i, ev, w=w, copies=copies, outs=outs):
            q, k, v = copies[i % 2]
            mark(ev, 0)
            A.prefill_fwd(q, k, v, causal=w.causal, scale=w.scale, out=outs[i % 2])
            mark(ev, 1)
        step_regions.append(Region(f"prefill_d{d}", launch, [(
            f"prefill_fwd_kernel<bf16,d{d},noncausal>", "prefill_fwd_kernel", "mfma", w.flops(), w.name,
            {"compulsory_bytes": w.io_bytes()})], finite(outs[0], w.name)))

    dec_info = None
    if want("step", "decode"):
        w = workloads.WORKLOADS[C4]
        copies = []
        for s in (0, 1):
            q, kc, vc, lens = workloads.decode_inputs(w, device=dev, salt=s)
            copies.append((q, kc, vc, lens.to(dev)))
        S = A.decode_num_splits(w.batch, w.hkv, w.max_kv_len)
        part = partials(w, S)
        out = torch.empty((w.batch, w.hq, w.d), dtype=torch.bfloat16, device=dev)
        total = int(copies[0][3].sum())

        def launch(i, ev, w=w, copies=copies, S=S, part=part, out=out):
            q, kc, vc, lens = copies[i % 2]
            mark(ev, 0)
            A.decode_splitk(q, kc, vc, lens, S, w.scale, partials=part)
            mark(ev, 1)
            A.merge_partials(*part, torch.bfloat16, out=out)
            mark(ev, 2)
        part_bytes = w.batch * w.hq * S * (w.d + 2) * 4.0
        dec_info = (w, S, w.kv_bytes(total))
        step_regions.append(Region("decode", launch, [
            ("decode_splitk_kernel<bf16,d128>", "decode_splitk_kernel", "hbm", w.kv_bytes(total), w.name,
             {"num_splits": S, "chunk": A.decode_chunk_len(w.max_kv_len, S)}),
            ("merge_partials_kernel<bf16,d128>", "merge_partials_kernel", "hbm", part_bytes, w.name,
             {"num_splits": S})], finite(out, w.name)))

    # ---- the causal GQA N=32768 prefill
    if want("prefill_causal_gqa"):
        w = workloads.WORKLOADS[C3]
        copies = [workloads.prefill_inputs(w, device=dev, salt=s) for s in (0, 1)]
        outs = [torch.empty_like(c[0]) for c in copies]

        def launch(i, ev, w=w, copies=copies, outs=outs):
            q, k, v = copies[i % 2]
            mark(ev, 0)
            A.prefill_fwd(q, k, v, causal=True, scale=w.scale, out=outs[i % 2])
            mark(ev, 1)
        other_regions.append(Region("prefill_causal_gqa", launch, [(
            "prefill_fwd_kernel<bf16,d128,causal>", "prefill_fwd_kernel", "mfma", w.flops(), w.name,
            {"compulsory_bytes": w.io_bytes()})], finite(outs[0], w.name)))

    # ---- the ragged batched decode (64 sequences, q x8)
    if want("decode_ragged"):
        w = workloads.WORKLOADS[C5]
        q, kc, vc, lens = workloads.decode_inputs(w, device=dev)
        lens_d = lens.to(dev)
        S = A.decode_num_splits(w.batch, w.hkv, w.max_kv_len)
        part = partials(w, S)
        out = torch.empty((w.batch, w.hq, w.d), dtype=torch.bfloat16, device=dev)
        total = int(lens.sum())

        def launch(i, ev, w=w, q=q, kc=kc, vc=vc, lens_d=lens_d, S=S, part=part, out=out):
            mark(ev, 0)
            A.decode_splitk(q, kc, vc, lens_d, S, w.scale, partials=part)
            mark(ev, 1)
            A.merge_partials(*part, torch.bfloat16, out=out)
            mark(ev, 2)
        part_bytes = w.batch * w.hq * S * (w.d + 2) * 4.0
        other_regions.append(Region("decode_ragged", launch, [
            ("decode_splitk_kernel<bf16,d128,ragged>", "decode_splitk_kernel", "hbm", w.kv_bytes(total), w.name,
             {"num_splits": S, "chunk": A.decode_chunk_len(w.max_kv_len, S), "sum_kv_len": total}),
            ("merge_partials_kernel<bf16,d128,ragged>", "merge_partials_kernel", "hbm", part_bytes, w.name,
             {"num_splits": S})], finite(out, w.name)))

    # ---- the one-head causal N=512 fp16 prefill (launch-bound)
    if want("prefill_small"):
        w = workloads.WORKLOADS[C1]
        copies = [workloads.prefill_inputs(w, device=dev, salt=s) for s in (0, 1)]
        outs = [torch.empty_like(c[0]) for c in copies]

        def launch(i, ev, w=w, copies=copies, outs=outs):
            q, k, v = copies[i % 2]
            mark(ev, 0)
            A.prefill_fwd(q, k, v, causal=True, scale=w.scale, out=outs[i % 2])
            mark(ev, 1)
        other_regions.append(Region("prefill_small", launch, [(
            "prefill_fwd_kernel<f16,d64,causal>", "prefill_fwd_kernel", "mfma", w.flops(), w.name,
            {"note": "2 workgroups on 256 CUs: launch-bound, timed for completeness"})], finite(outs[0], w.name)))

    # ---- next rows: paged decode, append batch, 4-bit decode
    if want("decode_paged"):
        w = workloads.WORKLOADS[C4]
        copies = []
        for s in (0, 1):
            q, kc, vc, lens = workloads.decode_inputs(w, device=dev, salt=s)
            kp, vp, table = workloads.paged_from_cache(kc, vc, lens, PAGE_SIZE, workloads.seed_for(w.name, "pages", s))
            del kc, vc
            copies.append((q, kp, vp, table.to(dev), lens.to(dev)))
        S = A.decode_num_splits(w.batch, w.hkv, copies[0][3].shape[1] * PAGE_SIZE)
        part = partials(w, S)
        out = torch.empty((w.batch, w.hq, w.d), dtype=torch.bfloat16, device=dev)
        total = int(copies[0][4].sum())

        def launch(i, ev, w=w, copies=copies, S=S, part=part, out=out):
            q, kp, vp, table, lens = copies[i % 2]
            mark(ev, 0)
            A.decode_splitk_paged(q, kp, vp, table, lens, S, w.scale, partials=part)
            mark(ev, 1)
            A.merge_partials(*part, torch.bfloat16, out=out)
            mark(ev, 2)
        other_regions.append(Region("decode_paged", launch, [
            (f"decode_splitk_kernel<bf16,d128,paged{PAGE_SIZE}>", "decode_splitk_kernel", "hbm", w.kv_bytes(total),
             f"{w.name} in {PAGE_SIZE}-row pages", {"num_splits": S}),
            ("merge_partials_kernel<bf16,d128>", "merge_partials_kernel", "hbm",
             w.batch * w.hq * S * (w.d + 2) * 4.0, w.name, {"num_splits": S})], finite(out, "paged decode")))

    if want("append"):
        w = workloads.WORKLOADS[APPEND]
        nq, nk = w.lengths()
        copies = []
        for s in (0, 1):
            q, k, v, cu_q, cu_k = workloads.varlen_inputs(w, device=dev, salt=s, nq=nq, nk=nk)
            copies.append((q, k, v, cu_q.to(dev), cu_k.to(dev)))
        outs = [torch.empty_like(c[0]) for c in copies]

        def launch(i, ev, w=w, copies=copies, outs=outs, nq=nq, nk=nk):
            q, k, v, cu_q, cu_k = copies[i % 2]
            mark(ev, 0)
            A.prefill_varlen_fwd(q, k, v, cu_q, cu_k, max(nq), max(nk), causal=w.causal, scale=w.scale,
                                 out=outs[i % 2])
            mark(ev, 1)
        other_regions.append(Region("append", launch, [(
            "prefill_fwd_kernel<bf16,d128,causal,varlen>", "prefill_fwd_kernel", "mfma", w.flops(nq, nk), w.name,
            {"queries": sum(nq), "keys": sum(nk)})], finite(outs[0], w.name)))

    if want("decode_q4"):
        w = workloads.WORKLOADS[C4]
        copies = []
        for s in (0, 1):
            q, kc, vc, lens = workloads.decode_inputs(w, device=dev, salt=s)
            kq, ks = A.kv_quantize_q4(kc, True)   # the library's own encoder writes the 4-bit cache
            vq, vs = A.kv_quantize_q4(vc, True)
            del kc, vc
            copies.append((q, kq, ks, vq, vs, lens.to(dev)))
        S = A.decode_q4_num_splits(w.batch, w.hkv, w.max_kv_len)
        part = partials(w, S)
        out = torch.empty((w.batch, w.hq, w.d), dtype=torch.bfloat16, device=dev)
        total = int(copies[0][5].sum())
        q4_bytes = 2.0 * w.hkv * total * (w.d // 2 + 4)  # codes + one fp32 scale per row, K and V

        def launch(i, ev, w=w, copies=copies, S=S, part=part, out=out):
            q, kq, ks, vq, vs, lens = copies[i % 2]
            mark(ev, 0)
            A.decode_splitk_q4(q, kq, ks, vq, vs, lens, True, S, w.scale, partials=part)
            mark(ev, 1)
            A.merge_partials(*part, torch.bfloat16, out=out)
            mark(ev, 2)
        other_regions.append(Region("decode_q4", launch, [
            ("decode_q4_kernel<bf16,d128,rotated>", "decode_q4_kernel", "hbm", q4_bytes,
             f"{w.name} as rotated 4-bit rows", {"num_splits": S, "bf16_equivalent_bytes": w.kv_bytes(total)}),
            ("merge_partials_kernel<bf16,d128>", "merge_partials_kernel", "hbm",
             w.batch * w.hq * S * (w.d + 2) * 4.0, w.name, {"num_splits": S})], finite(out, "4-bit decode")))

    if want("decode_q4_paged"):
        w = workloads.WORKLOADS[C4]
        copies = []
        for s in (0, 1):
            q, kc, vc, lens = workloads.decode_inputs(w, device=dev, salt=s)
            # 16-row pages in a seeded random order; the library's encoder writes each cache row
            # straight into its pool row (out_rows), as a serving loop appends rows to pages
            npg = w.max_kv_len // PAGE_SIZE
            gen = torch.Generator()
            gen.manual_seed(workloads.seed_for(w.name, "q4pages", s) & ((1 << 63) - 1))
            table = torch.randperm(w.batch * npg, generator=gen).to(torch.int32).reshape(w.batch, npg).to(dev)
            pos = torch.arange(w.max_kv_len, device=dev)
            kh = torch.arange(w.hkv, device=dev)[:, None]
            dest = ((table[:, pos // PAGE_SIZE].long()[:, None, :] * w.hkv + kh) * PAGE_SIZE
                    + pos % PAGE_SIZE).to(torch.int32).reshape(-1)
            pools = []
            for cache in (kc, vc):
                pc = torch.empty((w.batch * npg, w.hkv, PAGE_SIZE, w.d // 2), dtype=torch.uint8, device=dev)
                psc = torch.empty((w.batch * npg, w.hkv, PAGE_SIZE), dtype=torch.float32, device=dev)
                A.kv_quantize_q4(cache.reshape(-1, w.d), True, dest, pc.view(-1, w.d // 2), psc.view(-1))
                pools += [pc, psc]
            del kc, vc, dest
            copies.append((q, *pools, table, lens.to(dev)))
        S = A.decode_q4_num_splits(w.batch, w.hkv, w.max_kv_len)
        part = partials(w, S)
        out = torch.empty((w.batch, w.hq, w.d), dtype=torch.bfloat16, device=dev)
        total = int(copies[0][6].sum())
        q4_bytes = 2.0 * w.hkv * total * (w.d // 2 + 4)

        def launch(i, ev, w=w, copies=copies, S=S, part=part, out=out):
            q, kp, ksp, vp, vsp, table, lens = copies[i % 2]
            mark(ev, 0)
            A.decode_splitk_q4_paged(q, kp, ksp, vp, vsp, table, lens, True, S, w.scale, partials=part)
            mark(ev, 1)
            A.merge_partials(*part, torch.bfloat16, out=out)
            mark(ev, 2)
        other_regions.append(Region("decode_q4_paged", launch, [
            (f"decode_q4_kernel<bf16,d128,rotated,paged{PAGE_SIZE}>", "decode_q4_kernel", "hbm", q4_bytes,
             f"{w.name} as rotated 4-bit rows in {PAGE_SIZE}-row pages",
             {"num_splits": S, "bf16_equivalent_bytes": w.kv_bytes(total)}),
            ("merge_partials_kernel<bf16,d128>", "merge_partials_kernel", "hbm",
             w.batch * w.hq * S * (w.d + 2) * 4.0, w.name, {"num_splits": S})], finite(out, "paged 4-bit decode")))
    torch.cuda.synchronize()

    regions = step_regions + other_regions

    # ---- timing
    for reg in regions:
        run_region(torch, stream, reg, K, W, args.region_warmup_s)
        log(f"region {reg.name}: {reg.warm_launches} warm-up (at least {W} and {args.region_warmup_s} s), "
            f"{K} wall-clocked, {max(K, MIN_EVENT_LAUNCHES)} event-timed")

    kernels = []
    for reg in step_regions:
        kernels += kernel_records(reg, True)
    for reg in other_regions:
        kernels += kernel_records(reg, False)

    def region(name):
        return next((r for r in step_regions + other_regions if r.name == name), None)

    def wall_rate(reg, work, unit):
        if reg is None:
            return None
        rate = work * K / reg.wall_s / (1e12 if unit == "TFLOP/s" else 1e9)
        peak = PEAK_MFMA_BF16_TFLOPS if unit == "TFLOP/s" else PEAK_HBM_GBS
        return {"value": rate, "unit": unit, "frac_of_peak": rate / peak, "ms_per_call": reg.wall_s / K * 1e3}

    pre_regs = [r for r in step_regions if r.name.startswith("prefill")]
    pre_wall = sum(r.wall_s for r in pre_regs)
    pre_flops = sum(r.kernels[0][3] for r in pre_regs)
    dec_reg = region("decode")
    value = pre_flops * K / pre_wall / 1e12 if pre_regs else None

    in_step = [r for r in kernels if r["in_step"]]
    dominant = max(in_step or kernels, key=lambda r: r["avg_ms"])
    roofline = {k: dominant[k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic")}
    roofline["kernel"] = dominant["kernel"]
    roofline["avg_ms"] = dominant["avg_ms"]
    roofline["median_ms"] = dominant["median_ms"]

    def extra(name, work, unit, timed):
        reg = region(name)
        if reg is None:
            return None
        rec = wall_rate(reg, work(reg), unit)
        rec["timed"] = timed
        return rec

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": (pre_wall + (dec_reg.wall_s if dec_reg else 0.0)) / K * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": " + ".join([C2[0], C2[1], C4]),
            "prefill": [{"workload": n, "batch": 4, "hq": 32, "hkv": 32, "n": 4096, "d": d, "causal": False}
                        for n, d in zip(C2, (64, 128))],
            "decode": ({"workload": C4, "batch": 1, "hq": 32, "hkv": 8, "d": 128, "kv_len": 262144,
                        "num_splits": dec_info[1]} if dec_info else None),
        },
        "prefill_frac_of_mfma_peak": (value / PEAK_MFMA_BF16_TFLOPS) if value else None,
        "decode": extra("decode", lambda r: r.kernels[0][3], "GB/s",
                        "attn_decode_splitk + attn_merge_partials, wall clock"),
        "prefill_causal_gqa": extra("prefill_causal_gqa", lambda r: r.kernels[0][3], "TFLOP/s",
                                    "attn_prefill_fwd, wall clock, outside the step"),
        "decode_ragged": extra("decode_ragged", lambda r: r.kernels[0][3], "GB/s",
                               "attn_decode_splitk + attn_merge_partials, wall clock, outside the step"),
        "prefill_small": extra("prefill_small", lambda r: r.kernels[0][3], "TFLOP/s",
                               "attn_prefill_fwd, wall clock, outside the step (launch-bound)"),
        "decode_paged": extra("decode_paged", lambda r: r.kernels[0][3], "GB/s",
                              "attn_decode_splitk_paged + attn_merge_partials, wall clock, outside the step"),
        "append": extra("append", lambda r: r.kernels[0][3], "TFLOP/s",
                        "attn_prefill_varlen_fwd, wall clock, outside the step"),
        "decode_q4": extra("decode_q4", lambda r: r.kernels[0][3], "GB/s",
                           "attn_decode_splitk_q4 + attn_merge_partials, wall clock, outside the step"),
        "decode_q4_paged": extra("decode_q4_paged", lambda r: r.kernels[0][3], "GB/s",
                                 "attn_decode_splitk_q4_paged + attn_merge_partials, wall clock, outside the step"),
        "roofline": roofline,
        "kernels": kernels,
    }

    if only == "all" and not args.no_ceilings:
        ceil = measured_ceilings(torch, A._lib.load(), A._lib.check, stream)
        line["measured_ceilings"] = ceil
        for r in kernels:
            top = ceil["mfma_bf16_tflops"] if r["bound"] == "mfma" else ceil["hbm_read_gbs"]
            r["frac_of_measured"] = r["achieved"] / top
        roofline["frac_of_measured"] = dominant["frac_of_measured"]
    else:
        line["measured_ceilings"] = None

    if c2_inputs is not None and only == "all" and not args.no_cpu_baseline:
        log("cpu baseline (fp64 oracle on the host)")
        line["cpu_baseline"] = cpu_baseline(torch, workloads, dev, c2_inputs, args.cpu_seconds)
    else:
        line["cpu_baseline"] = None

    print(json.dumps(line), flush=True)
    return 0


# ---- rocprofv3 summaries (no GPU) ------------------------------------------------------------

def _read_csv(pattern):
    rows = []
    for path in sorted(glob.glob(pattern, recursive=True)):
        with open(path) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def summarize(base: str) -> int:
    """Print markdown tables from rocprofv3 output under ``base``: kernel
    statistics (``*kernel_stats.csv``) and counter collections
    (``*counter_collection.csv``, per kernel and counter: the median over
    dispatches of the per-dispatch sum)."""
    import collections

    stats = _read_csv(os.path.join(base, "**", "*kernel_stats.csv"))
    if stats:
        print("| kernel | calls | average (µs) | min (µs) | max (µs) | share of GPU time |")
        print("|---|---|---|---|---|---|")
        for r in stats:
            if "attn::" not in r["Name"]:
                continue
            name = r["Name"].split("(")[0].replace("void ", "")
            print(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                  f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f} % |")
    counters = _read_csv(os.path.join(base, "**", "*counter_collection.csv"))
    if counters:
        per = collections.defaultdict(lambda: collections.defaultdict(float))
        for r in counters:
            name = r["Kernel_Name"].split("(")[0].replace("void ", "")
            per[(name, r["Counter_Name"])][int(r["Dispatch_Id"])] += float(r["Counter_Value"])
        print("\n| kernel | counter | dispatches | median per dispatch |")
        print("|---|---|---|---|")
        for (name, counter), vals in sorted(per.items()):
            v = sorted(vals.values())
            print(f"| `{name}` | {counter} | {len(v)} | {v[len(v) // 2]:.6g} |")
    if not stats and not counters:
        print(f"no rocprofv3 csv output under {base}", file=sys.stderr)
        return 1
    return 0


def _per_dispatch(path_dir: str, kernel: str, counter: str):
    """Median over dispatches of one counter's per-dispatch sum for kernels whose
    name contains ``kernel``, and the number of dispatches."""
    import collections

    vals = collections.defaultdict(float)
    for r in _read_csv(os.path.join(path_dir, "**", "*counter_collection.csv")):
        if kernel in r["Kernel_Name"] and r["Counter_Name"] == counter:
            vals[int(r["Dispatch_Id"])] += float(r["Counter_Value"])
    v = sorted(vals.values())
    return (v[len(v) // 2], len(v)) if v else (None, 0)


def write_traffic(base: str) -> int:
    """HBM bytes per launch from ``rocprofv3 --pmc FETCH_SIZE`` and ``--pmc
    WRITE_SIZE`` runs: ``base/<region>_fetch`` and ``base/<region>_write`` hold
    the runs of ``bench.py --only <region>``, ``base/copy_fetch`` and
    ``base/copy_write`` those of ``bench.py --copy-calibration-mib 1024``.  Each
    counter is scaled by what it reads for the plain 1 GiB copy (1 GiB read,
    1 GiB written), and the record carries the kernel's source hash, so the
    bench reports it only while the kernel is unchanged."""
    copy_kib = float(1 << 20)
    cf, _ = _per_dispatch(os.path.join(base, "copy_fetch"), "copyBuffer", "FETCH_SIZE")
    cw, _ = _per_dispatch(os.path.join(base, "copy_write"), "copyBuffer", "WRITE_SIZE")
    if cf is None or cw is None:
        cf, _ = _per_dispatch(os.path.join(base, "copy_fetch"), "copy", "FETCH_SIZE")
        cw, _ = _per_dispatch(os.path.join(base, "copy_write"), "copy", "WRITE_SIZE")
    if cf is None or cw is None:
        print(f"no copy calibration under {base}", file=sys.stderr)
        return 1
    ff, fw = copy_kib / cf, copy_kib / cw
    try:
        with open(TRAFFIC_FILE) as fh:
            out = json.load(fh)
    except (OSError, ValueError):
        out = {"kernels": {}}
    out["about"] = ("HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE (KiB per dispatch, median over "
                    "dispatches), scaled by what the same counters read for a plain 1 GiB device copy; written by "
                    "bench.py --write-traffic.  bench.py reports a kernel's figure only while its source hash "
                    "matches source_sha.")
    out["command"] = ("cd /tmp && timeout -s KILL 90 rocprofv3 --pmc FETCH_SIZE|WRITE_SIZE --output-format csv "
                      "-d <dir>/<region>_fetch|_write -o run -- python <repo>/bench.py --no-cpu-baseline "
                      "--region-warmup-s 0 --only <region> --steps 2 --warmup 1 (calibration: -d <dir>/copy_fetch|copy_write ... "
                      "--copy-calibration-mib 1024 --steps 3); then python bench.py --write-traffic <dir>")
    out["calibration"] = {"copy_bytes": 1 << 30, "fetch_size_kib": cf, "write_size_kib": cw, "fetch_factor": ff,
                          "write_factor": fw}
    kernels = out.setdefault("kernels", {})
    for label, (rname, region) in ROCPROF_NAMES.items():
        if not os.path.isdir(os.path.join(base, region + "_fetch")):
            continue
        f, n1 = _per_dispatch(os.path.join(base, region + "_fetch"), rname, "FETCH_SIZE")
        w, n2 = _per_dispatch(os.path.join(base, region + "_write"), rname, "WRITE_SIZE")
        if f is None or w is None:
            continue
        src = label.split("<")[0]
        kernels[label] = {"fetch_size_kib": f, "write_size_kib": w, "dispatches": [n1, n2],
                          "fetch_bytes_per_launch": f * 1024 * ff, "write_bytes_per_launch": w * 1024 * fw,
                          "source_sha": source_sha(src)}
        print(f"{label}: {f * 1024 * ff / 1e6:.1f} MB read, {w * 1024 * fw / 1e6:.1f} MB written per launch")
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
    print(f"calibration factors: fetch {ff:.4f}, write {fw:.4f}")
    return 0


if __name__ == "__main__":
    sys.exit(main())

#!/usr/bin/env python3
"""Benchmark of the exact-attention hot path on one MI355X.

One step is one pass of the whole path over synthetic inputs already resident
in HBM:

* prefill forward on the non-causal batch-4, 32-head, N=4096 bf16 workload at
  d=64 and at d=128 (``attn_prefill_fwd``), and
* single-query split-K decode over one sequence's 262144-position bf16 cache
  with 32 query / 8 KV heads, d=128 (``attn_decode_splitk`` then
  ``attn_merge_partials``).

The prefill and decode halves are timed as two separately synchronised regions
of K steps each (wall clock, ``torch.cuda.synchronize`` on both sides), after W
untimed warm-up steps.  ``value`` is the prefill throughput in algorithmic
TFLOP/s (4·d FLOPs per visible query-key pair); the decode throughput in
algorithmic KV GB/s (every K and V byte read once) is reported beside it.  Each
kernel's average launch duration is taken with HIP events recorded on the
stream the kernels are launched on, around the launches of every fifth timed
step (an event pair around every launch would add about 10 µs of stream
overhead to each decode step's wall clock); the ``roofline`` object is for the
dominant (longest-running) kernel, ``kernels`` lists all of them.  Inputs
alternate between two copies so no launch finds the previous one's data in the
last-level cache.

After the step, the same decode is timed once more over a paged copy of the
cache (16-row pages in a seeded random order, ``attn_decode_splitk_paged`` then
``attn_merge_partials``) in a region of its own, and so is a packed append
batch (16 sequences of 256..2048 new queries on 0..16384 cached positions,
causal, ``attn_prefill_varlen_fwd``), and the decode over the cache encoded
as rotated 4-bit rows (``attn_decode_splitk_q4`` then ``attn_merge_partials``).
They are reported beside the step (``decode_paged``, ``append``,
``decode_q4`` and in ``kernels``) and are not part of ``value`` or
``ms_per_step``.

``measured_ceilings`` gives two rates measured on the same GPU in the same
run, with the library's measurement helpers (``include/attn_calibrate.h``): a
back-to-back bf16 MFMA loop and a streaming read of a 1 GiB buffer; each
kernel in ``kernels`` also carries ``frac_of_measured``, its rate against the
ceiling of its bound (``frac`` stays the fraction of the published peak).

``cpu_baseline`` times the fp64 oracle on a bounded sample of the same prefill
workload (whole heads until about ``--cpu-seconds`` have passed), on the host
cores, as a reported baseline only.

Prints exactly one JSON line on stdout.  Only one GPU is supported.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "prefill TFLOP/s and decode KV GB/s on 1 MI355X, each as % of roofline"
PEAK_MFMA_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0            # MI355X HBM3E peak
PREFILL = ["prefill_b4_h32_n4096_d64_bf16", "prefill_b4_h32_n4096_d128_bf16"]
DECODE = "decode_b1_hq32_hkv8_d128_len262144_bf16"
PAGE_SIZE = 16
EVENT_EVERY = 5                  # timed steps whose launches are bracketed by HIP events
APPEND = "append_causal_b16_hq32_hkv8_d128_q256to2048_past0to16384_bf16"
CSRC = os.path.join(ROOT, "exact_attention_flashattention_amd", "csrc")
KERNEL_SOURCES = {
    "prefill_fwd_kernel": ["prefill_fwd.hip", "device_common.hpp"],
    "decode_splitk_kernel": ["decode_splitk.hip", "device_common.hpp"],
    "merge_partials_kernel": ["merge_partials.hip", "device_common.hpp"],
    "decode_q4_kernel": ["decode_q4.hip", "device_common.hpp"],
    "quantize_q4_kernel": ["quantize_q4.hip", "device_common.hpp"],
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")


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


def cpu_baseline(inputs, w, seconds: float):
    """The oracle, untuned, on whole heads of the d=128 prefill workload until
    ``seconds`` of CPU time have passed."""
    import numpy as np
    import oracle

    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"),
                      default=1)
    except Exception:  # pragma: no cover
        threads = 1
    q, k, v = inputs
    g = w.hq // w.hkv
    done, flops, elapsed = 0, 0.0, 0.0
    per_head = 4.0 * w.d * w.n * w.n
    for b in range(w.batch):
        for h in range(w.hq):
            qh = q[b, h].float().cpu().double().numpy()
            kh = k[b, h // g].float().cpu().double().numpy()
            vh = v[b, h // g].float().cpu().double().numpy()
            t0 = time.perf_counter()
            oracle.attention(qh[None, None], kh[None, None], vh[None, None], w.scale, w.causal)
            elapsed += time.perf_counter() - t0
            done += 1
            flops += per_head
            if elapsed >= seconds:
                break
        if elapsed >= seconds:
            break
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} of {w.batch * w.hq} (batch, head) slices of {w.name}, whole rows, fp64 numpy; "
                      f"{elapsed:.1f} s; host {cpu_model()}, {os.cpu_count()} logical CPUs"}


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


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the measured MFMA-loop and streaming-read ceilings")
    ap.add_argument("--only", choices=["all", "prefill_d64", "prefill_d128", "decode", "decode_paged", "append", "decode_q4"], default="all",
                    help="run only one kernel family (for profiler runs)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="instead of the bench, run plain device copies of this many MiB (counter calibration)")
    args = ap.parse_args()

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
    run_prefill = [n for n in PREFILL if args.only in ("all", "prefill_d" + n.split("_d")[1].split("_")[0])]
    run_decode = args.only in ("all", "decode")
    run_paged = args.only in ("all", "decode_paged")
    run_append = args.only in ("all", "append")
    run_q4 = args.only in ("all", "decode_q4")

    # ---- inputs (two copies each), outputs and workspaces: all allocated before timing
    pre = []
    for name in run_prefill:
        w = workloads.WORKLOADS[name]
        copies = [workloads.prefill_inputs(w, device=dev, salt=s) for s in (0, 1)]
        outs = [torch.empty_like(c[0]) for c in copies]
        pre.append((w, copies, outs))
    dec = None
    if run_decode:
        w = workloads.WORKLOADS[DECODE]
        copies = []
        for s in (0, 1):
            q, kc, vc, lens = workloads.decode_inputs(w, device=dev, salt=s)
            copies.append((q, kc, vc, lens.to(dev)))
        S = A.decode_num_splits(w.batch, w.hkv, w.max_kv_len)
        part = (torch.empty((w.batch, w.hq, S), dtype=torch.float32, device=dev),
                torch.empty((w.batch, w.hq, S), dtype=torch.float32, device=dev),
                torch.empty((w.batch, w.hq, S, w.d), dtype=torch.float32, device=dev))
        out = torch.empty((w.batch, w.hq, w.d), dtype=torch.bfloat16, device=dev)
        total_len = int(sum(int(c[3].sum()) for c in copies[:1]))
        dec = (w, copies, S, part, out, total_len)
    pag = None
    if run_paged:
        w = workloads.WORKLOADS[DECODE]
        copies = []
        for s in (0, 1):
            q, kc, vc, lens = workloads.decode_inputs(w, device=dev, salt=s)
            kp, vp, table = workloads.paged_from_cache(kc, vc, lens, PAGE_SIZE, workloads.seed_for(w.name, "pages", s))
            del kc, vc
            copies.append((q, kp, vp, table.to(dev), lens.to(dev)))
        S = A.decode_num_splits(w.batch, w.hkv, copies[0][3].shape[1] * PAGE_SIZE)
        part = (torch.empty((w.batch, w.hq, S), dtype=torch.float32, device=dev),
                torch.empty((w.batch, w.hq, S), dtype=torch.float32, device=dev),
                torch.empty((w.batch, w.hq, S, w.d), dtype=torch.float32, device=dev))
        out = torch.empty((w.batch, w.hq, w.d), dtype=torch.bfloat16, device=dev)
        pag = (w, copies, S, part, out, int(copies[0][4].sum()))
    app = None
    if run_append:
        w = workloads.WORKLOADS[APPEND]
        nq, nk = w.lengths()
        copies = []
        for s in (0, 1):
            q, k, v, cu_q, cu_k = workloads.varlen_inputs(w, device=dev, salt=s, nq=nq, nk=nk)
            copies.append((q, k, v, cu_q.to(dev), cu_k.to(dev)))
        outs = [torch.empty_like(c[0]) for c in copies]
        app = (w, copies, outs, nq, nk)
    dq4 = None
    if run_q4:
        w = workloads.WORKLOADS[DECODE]
        copies = []
        for s in (0, 1):
            q, kq, ks, vq, vs, lens = workloads.decode_q4_inputs(w, True, device=dev, salt=s)
            copies.append((q, kq, ks, vq, vs, lens.to(dev)))
        S = A.decode_num_splits(w.batch, w.hkv, w.max_kv_len)
        part = (torch.empty((w.batch, w.hq, S), dtype=torch.float32, device=dev),
                torch.empty((w.batch, w.hq, S), dtype=torch.float32, device=dev),
                torch.empty((w.batch, w.hq, S, w.d), dtype=torch.float32, device=dev))
        out = torch.empty((w.batch, w.hq, w.d), dtype=torch.bfloat16, device=dev)
        dq4 = (w, copies, S, part, out, int(copies[0][5].sum()))
    torch.cuda.synchronize()

    def prefill_step(i, ev=None):
        for j, (w, copies, outs) in enumerate(pre):
            q, k, v = copies[i % 2]
            if ev is not None:
                ev[j][0].record(stream)
            A.prefill_fwd(q, k, v, causal=w.causal, scale=w.scale, out=outs[i % 2])
            if ev is not None:
                ev[j][1].record(stream)

    def decode_step(i, ev=None):
        w, copies, S, part, out, _ = dec
        q, kc, vc, lens = copies[i % 2]
        if ev is not None:
            ev[0].record(stream)
        A.decode_splitk(q, kc, vc, lens, S, w.scale, partials=part)
        if ev is not None:
            ev[1].record(stream)
        A.merge_partials(*part, torch.bfloat16, out=out)
        if ev is not None:
            ev[2].record(stream)

    def paged_step(i, ev=None):
        w, copies, S, part, out, _ = pag
        q, kp, vp, table, lens = copies[i % 2]
        if ev is not None:
            ev[0].record(stream)
        A.decode_splitk_paged(q, kp, vp, table, lens, S, w.scale, partials=part)
        if ev is not None:
            ev[1].record(stream)
        A.merge_partials(*part, torch.bfloat16, out=out)
        if ev is not None:
            ev[2].record(stream)

    def append_step(i, ev=None):
        w, copies, outs, nq, nk = app
        q, k, v, cu_q, cu_k = copies[i % 2]
        if ev is not None:
            ev[0].record(stream)
        A.prefill_varlen_fwd(q, k, v, cu_q, cu_k, max(nq), max(nk), causal=w.causal, scale=w.scale, out=outs[i % 2])
        if ev is not None:
            ev[1].record(stream)

    def q4_step(i, ev=None):
        w, copies, S, part, out, _ = dq4
        q, kq, ks, vq, vs, lens = copies[i % 2]
        if ev is not None:
            ev[0].record(stream)
        A.decode_splitk_q4(q, kq, ks, vq, vs, lens, True, S, w.scale, partials=part)
        if ev is not None:
            ev[1].record(stream)
        A.merge_partials(*part, torch.bfloat16, out=out)
        if ev is not None:
            ev[2].record(stream)

    def events(n):
        return [torch.cuda.Event(enable_timing=True) for _ in range(n)]

    def timed_with_events():
        return range(0, K, EVENT_EVERY)

    result_kernels = []
    pre_wall = dec_wall = 0.0
    pre_flops = sum(w.flops() for w, _, _ in pre)

    # ---- prefill region
    if pre:
        for i in range(W):
            prefill_step(i)
        torch.cuda.synchronize()
        ev = {i: [events(2) for _ in pre] for i in timed_with_events()}
        t0 = time.perf_counter()
        for i in range(K):
            prefill_step(i, ev.get(i))
        torch.cuda.synchronize()
        pre_wall = time.perf_counter() - t0
        for j, (w, _, outs) in enumerate(pre):
            ms = sum(e[j][0].elapsed_time(e[j][1]) for e in ev.values()) / len(ev)
            tflops = w.flops() / (ms * 1e-3) / 1e12
            if not torch.isfinite(outs[0]).all():
                raise RuntimeError(f"non-finite prefill output on {w.name}")
            label = f"prefill_fwd_kernel<bf16,d{w.d},{'causal' if w.causal else 'noncausal'}>"
            traffic = measured_traffic(label, "prefill_fwd_kernel")
            result_kernels.append({
                "kernel": label, "workload": w.name, "avg_ms": ms, "bound": "mfma", "achieved": tflops,
                "peak": PEAK_MFMA_BF16_TFLOPS, "unit": "TFLOP/s", "frac": tflops / PEAK_MFMA_BF16_TFLOPS,
                "traffic": traffic, "algorithmic_flops": w.flops(), "compulsory_bytes": w.io_bytes()})

    # ---- decode region
    if dec:
        w, copies, S, part, out, total_len = dec
        for i in range(W):
            decode_step(i)
        torch.cuda.synchronize()
        ev = {i: events(3) for i in timed_with_events()}
        t0 = time.perf_counter()
        for i in range(K):
            decode_step(i, ev.get(i))
        torch.cuda.synchronize()
        dec_wall = time.perf_counter() - t0
        if not torch.isfinite(out).all():
            raise RuntimeError("non-finite decode output")
        kv_bytes = w.kv_bytes(total_len)
        ms_split = sum(e[0].elapsed_time(e[1]) for e in ev.values()) / len(ev)
        ms_merge = sum(e[1].elapsed_time(e[2]) for e in ev.values()) / len(ev)
        gbs = kv_bytes / (ms_split * 1e-3) / 1e9
        result_kernels.append({
            "kernel": "decode_splitk_kernel<bf16,d128>", "workload": w.name, "avg_ms": ms_split, "bound": "hbm",
            "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
            "traffic": measured_traffic("decode_splitk_kernel<bf16,d128>", "decode_splitk_kernel"),
            "algorithmic_bytes": kv_bytes, "num_splits": S,
            "chunk": A.decode_chunk_len(w.max_kv_len, S)})
        part_bytes = 2.0 * w.batch * w.hq * S * (w.d + 2) * 4
        result_kernels.append({
            "kernel": "merge_partials_kernel<bf16,d128>", "workload": w.name, "avg_ms": ms_merge, "bound": "hbm",
            "achieved": part_bytes / 2 / (ms_merge * 1e-3) / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": part_bytes / 2 / (ms_merge * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "traffic": measured_traffic("merge_partials_kernel<bf16,d128>", "merge_partials_kernel"),
            "algorithmic_bytes": part_bytes / 2})

    # ---- paged decode region (reported beside the step)
    paged_line = None
    if pag:
        w, copies, S, part, out, total_len = pag
        for i in range(W):
            paged_step(i)
        torch.cuda.synchronize()
        ev = {i: events(3) for i in timed_with_events()}
        t0 = time.perf_counter()
        for i in range(K):
            paged_step(i, ev.get(i))
        torch.cuda.synchronize()
        pag_wall = time.perf_counter() - t0
        if not torch.isfinite(out).all():
            raise RuntimeError("non-finite paged decode output")
        kv_bytes = w.kv_bytes(total_len)
        ms_split = sum(e[0].elapsed_time(e[1]) for e in ev.values()) / len(ev)
        gbs = kv_bytes / (ms_split * 1e-3) / 1e9
        label = f"decode_splitk_kernel<bf16,d128,paged{PAGE_SIZE}>"
        result_kernels.append({
            "kernel": label, "workload": f"{w.name} in {PAGE_SIZE}-row pages", "avg_ms": ms_split,
            "bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
            "traffic": measured_traffic(label, "decode_splitk_kernel"), "algorithmic_bytes": kv_bytes,
            "num_splits": S, "in_step": False})
        paged_line = {"value": kv_bytes * K / pag_wall / 1e9, "unit": "GB/s",
                      "frac_of_hbm_peak": kv_bytes * K / pag_wall / 1e9 / PEAK_HBM_GBS, "page_size": PAGE_SIZE,
                      "timed": "attn_decode_splitk_paged + attn_merge_partials, wall clock, outside the step"}

    # ---- append (varlen prefill) region (reported beside the step)
    append_line = None
    if app:
        w, copies, outs, nq, nk = app
        for i in range(W):
            append_step(i)
        torch.cuda.synchronize()
        ev = {i: events(2) for i in timed_with_events()}
        t0 = time.perf_counter()
        for i in range(K):
            append_step(i, ev.get(i))
        torch.cuda.synchronize()
        app_wall = time.perf_counter() - t0
        if not torch.isfinite(outs[0]).all():
            raise RuntimeError("non-finite append output")
        flops = w.flops(nq, nk)
        ms = sum(e[0].elapsed_time(e[1]) for e in ev.values()) / len(ev)
        tflops = flops / (ms * 1e-3) / 1e12
        label = "prefill_fwd_kernel<bf16,d128,causal,varlen>"
        result_kernels.append({
            "kernel": label, "workload": w.name, "avg_ms": ms, "bound": "mfma", "achieved": tflops,
            "peak": PEAK_MFMA_BF16_TFLOPS, "unit": "TFLOP/s", "frac": tflops / PEAK_MFMA_BF16_TFLOPS,
            "traffic": measured_traffic(label, "prefill_fwd_kernel"), "algorithmic_flops": flops,
            "in_step": False})
        append_line = {"value": flops * K / app_wall / 1e12, "unit": "TFLOP/s",
                       "frac_of_mfma_peak": flops * K / app_wall / 1e12 / PEAK_MFMA_BF16_TFLOPS,
                       "queries": sum(nq), "keys": sum(nk),
                       "timed": "attn_prefill_varlen_fwd, wall clock, outside the step"}

    # ---- 4-bit cache decode region (reported beside the step)
    q4_line = None
    if dq4:
        w, copies, S, part, out, total_len = dq4
        for i in range(W):
            q4_step(i)
        torch.cuda.synchronize()
        ev = {i: events(3) for i in timed_with_events()}
        t0 = time.perf_counter()
        for i in range(K):
            q4_step(i, ev.get(i))
        torch.cuda.synchronize()
        q4_wall = time.perf_counter() - t0
        if not torch.isfinite(out).all():
            raise RuntimeError("non-finite 4-bit decode output")
        q4_bytes = 2.0 * w.hkv * total_len * (w.d // 2 + 4)  # codes + one fp32 scale per row, K and V
        ms_split = sum(e[0].elapsed_time(e[1]) for e in ev.values()) / len(ev)
        gbs = q4_bytes / (ms_split * 1e-3) / 1e9
        label = "decode_q4_kernel<bf16,d128,rotated>"
        result_kernels.append({
            "kernel": label, "workload": f"{w.name} as rotated 4-bit rows", "avg_ms": ms_split, "bound": "hbm",
            "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
            "traffic": measured_traffic(label, "decode_q4_kernel"), "algorithmic_bytes": q4_bytes,
            "num_splits": S, "in_step": False})
        q4_line = {"value": q4_bytes * K / q4_wall / 1e9, "unit": "GB/s",
                   "frac_of_hbm_peak": q4_bytes * K / q4_wall / 1e9 / PEAK_HBM_GBS,
                   "bf16_equivalent_gbs": w.kv_bytes(total_len) * K / q4_wall / 1e9,
                   "timed": "attn_decode_splitk_q4 + attn_merge_partials, wall clock, outside the step"}

    dominant = max([r for r in result_kernels if r.get("in_step", True)] or result_kernels, key=lambda r: r["avg_ms"])
    roofline = {k: dominant[k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic")}
    roofline["kernel"] = dominant["kernel"]

    value = pre_flops * K / pre_wall / 1e12 if pre else None
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": (pre_wall + dec_wall) / K * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": " + ".join([w.name for w, _, _ in pre] + ([dec[0].name] if dec else [])),
            "prefill": [{"workload": w.name, "batch": w.batch, "hq": w.hq, "hkv": w.hkv, "n": w.n, "d": w.d,
                         "causal": w.causal} for w, _, _ in pre],
            "decode": ({"workload": dec[0].name, "batch": dec[0].batch, "hq": dec[0].hq, "hkv": dec[0].hkv,
                        "d": dec[0].d, "kv_len": dec[0].max_kv_len, "num_splits": dec[2]} if dec else None),
        },
        "prefill_frac_of_mfma_peak": (value / PEAK_MFMA_BF16_TFLOPS) if value else None,
        "decode": ({"value": dec[0].kv_bytes(dec[5]) * K / dec_wall / 1e9, "unit": "GB/s",
                    "frac_of_hbm_peak": dec[0].kv_bytes(dec[5]) * K / dec_wall / 1e9 / PEAK_HBM_GBS,
                    "timed": "attn_decode_splitk + attn_merge_partials, wall clock"} if dec else None),
        "decode_paged": paged_line,
        "append": append_line,
        "decode_q4": q4_line,
        "roofline": roofline,
        "kernels": result_kernels,
    }

    if args.only == "all" and not args.no_ceilings:
        ceil = measured_ceilings(torch, A._lib.load(), A._lib.check, stream)
        line["measured_ceilings"] = ceil
        for r in result_kernels:
            top = ceil["mfma_bf16_tflops"] if r["bound"] == "mfma" else ceil["hbm_read_gbs"]
            r["frac_of_measured"] = r["achieved"] / top
    else:
        line["measured_ceilings"] = None

    if pre and not args.no_cpu_baseline:
        w, copies, _ = pre[-1]
        line["cpu_baseline"] = cpu_baseline(copies[0], w, args.cpu_seconds)
    else:
        line["cpu_baseline"] = None

    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

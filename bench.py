#!/usr/bin/env python3
"""Benchmark of the fused attention hot path on one MI355X.

One step = fa_fwd followed by the backward (every step of the forward and
the backward path) on the bwd workload: B=1, H=16, Sq=Sk=4096, d=128,
causal, bf16 inputs drawn by workloads.py (seed 5), O and LSE taken from
fa_fwd.  The backward is the five-product form (--bwd ds, the default:
fa_bwd_ds, enqueued as its three launches PREPARE, DKDV, DQ through
fa_bwd_ds_phase) or the split form (--bwd split: fa_bwd's two launches,
PREPARE | DQ, whose dQ kernel also forms the row terms, then DKDV), with HIP
events between the launches, on the stream the kernels run on, so each
kernel's average duration is measured inside the timed region; the form not
in the step is timed beside it.  Inputs and outputs are resident in device
memory before timing starts.

Printed: ONE JSON line with the throughput in TFLOP/s (counted FLOPs:
forward 4*B*H*S^2*d, backward 10*B*H*S^2*d, causal counts half), its share
of the MI355X dense bf16 MFMA peak (2516.6 TFLOP/s = 256 CUs x 2.4 GHz x 4096
FLOP/clk), a roofline entry for the dominant kernel, the CPU oracle timed on
a bounded sample of the same workload, and per-kernel / per-workload
details (including the long causal forward, B=1 H=16 S=8192 d=128).

Before the W warmup steps the step runs untimed for --warm-seconds (default
1 s) so that the GPU clocks have reached their sustained level; each forward
sweep workload is warmed the same way for a third of that.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--warm-seconds T]
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA, 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_FP8_TFLOPS = 5033.2      # MI355X dense fp8 MFMA, twice the bf16 rate
PEAK_FP4_TFLOPS = 10066.3     # MI355X dense fp4 MFMA, four times the bf16 rate
# the MXFP4 forward: half its counted FLOPs (S = Q K^T) at the fp4 rate, half
# (P V) at the fp8 rate -> the time-weighted peak of the mix
PEAK_MXFP4_MIX_TFLOPS = 1.0 / (0.5 / PEAK_FP4_TFLOPS + 0.5 / PEAK_FP8_TFLOPS)
PEAK_HBM_GBS = 8000.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--warm-seconds", type=float, default=1.0,
                   help="untimed run of the step before the warmup steps, so the GPU clocks "
                        "reach their sustained level (each forward sweep workload gets a third)")
    p.add_argument("--workload", type=int, default=5, help="workload id in workloads.WORKLOADS")
    p.add_argument("--tau", type=float, default=8.0)
    p.add_argument("--emu", type=float, default=0.0)
    p.add_argument("--deterministic", type=int, default=0)
    p.add_argument("--bwd", choices=("ds", "split"), default="ds",
                   help="backward of the step: five-product (fa_bwd_ds) or split by output (fa_bwd)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extra", action="store_true", help="skip the per-workload forward sweep")
    p.add_argument("--cpu-seconds", type=float, default=20.0, help="budget of the oracle sample")
    p.add_argument("--fwd-only", action="store_true")
    p.add_argument("--reps", type=int, default=0, help="only run K steps (for profilers), print nothing else")
    p.add_argument("--copy-mib", type=int, default=0,
                   help="with --reps: first run --reps plain device copies of this many MiB "
                        "(a known byte count that scales the HBM counters)")
    p.add_argument("--fp8", action="store_true",
                   help="with --reps and --fwd-only: run the e4m3 forward on the quantised workload")
    p.add_argument("--mxfp4", action="store_true",
                   help="with --reps and --fwd-only: run the MXFP4 forward (MXFP4 Q, K; e4m3 V)")
    p.add_argument("--fp8-blocks", action="store_true",
                   help="with --reps and --fwd-only: run the e4m3 forward with one factor per 128-row block")
    return p.parse_args()


class ClockSampler:
    """Samples the GPU's shader (GFX) clock every 20 ms from a side thread
    through the amdsmi library while the step runs (the sustained warm-up and
    the timed steps); mean / min / max in MHz, or None where the library or
    the device does not report it."""

    def __init__(self):
        import threading
        self.samples, self._stop = [], threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _run(self):
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            try:
                h = amdsmi.amdsmi_get_processor_handles()[0]
                while not self._stop.is_set():
                    self.samples.append(float(amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.GFX)["clk"]))
                    time.sleep(0.02)
            finally:
                amdsmi.amdsmi_shut_down()
        except Exception:
            pass

    def __enter__(self):
        self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._thread.join(timeout=5)

    def summary(self):
        s = self.samples
        if not s:
            return None
        # the warm-up synchronises between batches, so some samples catch the
        # clock dropping while the GPU waits: the median is taken over the
        # samples at 1 GHz or more (the GPU at work)
        busy = sorted(x for x in s if x >= 1000.0)
        return {"busy_median_mhz": busy[len(busy) // 2] if busy else None, "max_mhz": max(s),
                "busy_samples": len(busy), "samples": len(s),
                "source": "amdsmi GFX clock, sampled every 20 ms during the warm-up and the timed steps"}


def warm_gpu(fn, seconds):
    """Call fn() repeatedly for about `seconds` of wall time (untimed).  Under
    sustained load the MI355X shader clock settles within a fraction of a
    second; timing a cold GPU reads up to ~15 % slow."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()


def time_calls(fn, n, warmup, warm_s=0.0):
    """Mean milliseconds of fn() over n calls, HIP events on the current stream."""
    import torch
    warm_gpu(fn, warm_s)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


# the source file of each kernel; every kernel also depends on the shared headers
KERNEL_SOURCE = {"fwd_kernel": "fa_fwd.hip", "bwd_prep_kernel": "fa_bwd.hip", "bwd_dq_kernel": "fa_bwd.hip",
                 "bwd_dkdv_kernel": "fa_bwd.hip", "bwd_dkdv_kernel_ds": "fa_bwd.hip",
                 "bwd_dq_ds_kernel": "fa_bwd.hip", "merge_kernel": "fa_merge.hip", "fwd8_kernel": "fa_fwd8.hip"}


def kernel_sources_sha256(kernel):
    """Hash of the HIP sources `kernel` is built from: its own .hip file and
    the shared headers (ties a counter summary in profiles/ to the kernel
    version it measured)."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "exact_attention_50_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hpp", ".h")) or f == KERNEL_SOURCE[kernel]:
            h.update(f.encode())
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()


def read_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from profiles/traffic_<kernel>_<workload>.md
    (FETCH_SIZE + WRITE_SIZE counters scaled by a plain copy of known size), or
    None when no summary exists or the kernels changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and line.strip().startswith("- "):
            key, val = line.strip()[2:].split(":", 1)
            fields[key.strip()] = val.strip().strip("`")
    if fields.get("source_sha256") != kernel_sources_sha256(kernel):
        return None
    try:
        return int(float(fields["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, budget_s):
    """The float64 oracle (fwd + bwd) on whole heads of the workload, until the
    time budget is used; returns TFLOP/s of the same counted FLOPs."""
    import numpy as np
    from oracle import attention_backward, attention_forward
    from workloads import workload_inputs
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = 1
    done, t_total = 0, 0.0
    flops_per_head = (w.flops("fwd") + (w.flops("bwd") if w.kind == "bwd" else 0)) / (w.B * w.H)
    for h in range(w.H):
        ins = workload_inputs(w, heads=(h, h + 1))
        t0 = time.perf_counter()
        attention_forward(ins[0][:1], ins[1][:1], ins[2][:1], w.scale, w.causal)
        if w.kind == "bwd":
            attention_backward(ins[0][:1], ins[1][:1], ins[2][:1], ins[3][:1], w.scale, w.causal)
        t_total += time.perf_counter() - t0
        done += 1
        if t_total >= budget_s:
            break
    return {"value": round(flops_per_head * done / t_total / 1e12, 6), "unit": "TFLOP/s",
            "cores": int(threads), "kind": "oracle",
            "sample": f"{done} of {w.B * w.H} (b,h) heads of {w.name}, float64 NumPy "
                      f"{'fwd+bwd' if w.kind == 'bwd' else 'fwd'}, {t_total:.1f} s; "
                      f"GEMMs on {threads} BLAS threads, exp/max single-threaded; "
                      f"host has {len(os.sched_getaffinity(0))} usable cores"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the kernels are "
              "single-GPU and the multi-GPU sharding is a design note, not a built path.", file=sys.stderr)
        sys.exit(2)
    import torch
    import exact_attention_50_amd as fa
    from workloads import WORKLOADS, workload_inputs

    dev = "cuda:0"
    torch.cuda.set_device(0)
    w = WORKLOADS[args.workload]
    ins = [t.to(dev) for t in workload_inputs(w)]
    q, k, v = ins[:3]
    B, H, Sq, d = q.shape
    Sk = k.shape[2]
    do = ins[3] if len(ins) > 3 else torch.randn_like(q)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(max(16, fa.fa_bwd_workspace_bytes(B, H, Sq, Sk, d, w.causal, args.deterministic)),
                     dtype=torch.uint8, device=dev)
    do_bwd = not args.fwd_only
    ws_ds = None
    if do_bwd:
        ws_ds = torch.empty(fa.fa_bwd_ds_workspace_bytes(B, H, Sq, Sk, d, w.causal, args.deterministic),
                            dtype=torch.uint8, device=dev)

    def fwd():
        fa.fa_fwd(q, k, v, o, lse, causal=w.causal, scale=w.scale, tau=args.tau, emu_frac=args.emu)

    def bwd_split(det=args.deterministic):
        fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, ws, causal=w.causal, scale=w.scale, deterministic=bool(det))

    def bwd_ds(det=args.deterministic):
        fa.fa_bwd_ds(q, k, v, o, lse, do, dq, dk, dv, ws_ds, causal=w.causal, scale=w.scale,
                     deterministic=bool(det))

    bwd = bwd_ds if args.bwd == "ds" else bwd_split

    if args.reps:
        # profiler mode: optional plain copies of known size (to scale HBM
        # counters), then K steps; prints one line and nothing else
        if args.fp8:
            if do_bwd:
                sys.exit("--fp8 profiles the forward only: add --fwd-only")
            from workloads import quantise_e4m3
            (q8, qs), (k8, ks), (v8, vs) = (quantise_e4m3(t.cpu()) for t in (q, k, v))
            q8, k8, v8 = q8.to(dev), k8.to(dev), v8.to(dev)

            def fwd():
                fa.fa_fwd_fp8(q8, k8, v8, o, lse, qs, ks, vs, causal=w.causal, scale=w.scale, tau=args.tau)
        elif args.fp8_blocks:
            if do_bwd:
                sys.exit("--fp8-blocks profiles the forward only: add --fwd-only")
            from workloads import quantise_e4m3_blocks
            (qb8, qbf), (kb8, kbf), (vb8, vbf) = (quantise_e4m3_blocks(t.cpu()) for t in (q, k, v))
            qb8, kb8, vb8, qbf, kbf, vbf = (t.to(dev) for t in (qb8, kb8, vb8, qbf, kbf, vbf))

            def fwd():
                fa.fa_fwd_fp8_blocks(qb8, kb8, vb8, qbf, kbf, vbf, o, lse, causal=w.causal, scale=w.scale,
                                     tau=args.tau)
        elif args.mxfp4:
            if do_bwd:
                sys.exit("--mxfp4 profiles the forward only: add --fwd-only")
            from workloads import quantise_e4m3, quantise_mxfp4
            q4, q4s = (t.to(dev) for t in quantise_mxfp4(q.cpu()))
            k4, k4s = (t.to(dev) for t in quantise_mxfp4(k.cpu()))
            v8, vs = quantise_e4m3(v.cpu())
            v8 = v8.to(dev)

            def fwd():
                fa.fa_fwd_mxfp4(q4, q4s, k4, k4s, v8, o, lse, vs, causal=w.causal, scale=w.scale, tau=args.tau)
        if args.copy_mib:
            src = torch.ones(args.copy_mib * 2**20 // 4, dtype=torch.float32, device=dev)
            dst = torch.empty_like(src)
            for _ in range(args.reps):
                dst.copy_(src)
            torch.cuda.synchronize()
            del src, dst
        for _ in range(args.reps):
            fwd()
            if do_bwd:
                bwd()
        torch.cuda.synchronize()
        print(f"ran {args.reps} steps of {w.name}" + (" (e4m3 forward)" if args.fp8 else "") +
              (" (MXFP4 forward)" if args.mxfp4 else "") +
              (" (e4m3 forward, block factors)" if args.fp8_blocks else "") +
              (f" after {args.reps} copies of {args.copy_mib} MiB" if args.copy_mib else ""), flush=True)
        return

    def bwd_phase(ph):
        fa.fa_bwd_phase(ph, q, k, v, o, lse, do, dq, dk, dv, ws, causal=w.causal, scale=w.scale,
                        deterministic=bool(args.deterministic))

    def bwd_ds_phase(ph):
        fa.fa_bwd_ds_phase(ph, q, k, v, o, lse, do, dq, dk, dv, ws_ds, causal=w.causal, scale=w.scale,
                           deterministic=bool(args.deterministic))

    # the step, kernel by kernel, as the backward call launches it.  Five
    # products: PREPARE (row terms), DKDV (dK, dV and dS), DQ (dQ from dS).
    # Split: PREPARE and DQ in one call (the dQ kernel forms the row terms
    # D_i, LSE_i log2(e) itself), then DKDV
    parts = [("fwd_kernel", fwd)]
    if do_bwd and args.bwd == "ds":
        parts += [("bwd_prep_kernel", lambda: bwd_ds_phase(fa.FA_BWD_PREPARE)),
                  ("bwd_dkdv_kernel_ds", lambda: bwd_ds_phase(fa.FA_BWD_DKDV)),
                  ("bwd_dq_ds_kernel", lambda: bwd_ds_phase(fa.FA_BWD_DQ))]
    elif do_bwd:
        parts += [("bwd_dq_kernel", lambda: bwd_phase(fa.FA_BWD_PREPARE | fa.FA_BWD_DQ)),
                  ("bwd_dkdv_kernel", lambda: bwd_phase(fa.FA_BWD_DKDV))]

    # ---- clock warm-up and W warmup steps, then exactly K timed steps, then
    # K steps with events between the kernels
    def step():
        for _, fn in parts:
            fn()

    sclk = ClockSampler()
    sclk.__enter__()
    warm_gpu(step, args.warm_seconds)
    for _ in range(args.warmup):
        for _, fn in parts:
            fn()
    torch.cuda.synchronize()
    # the K timed steps: one event before the first and one after the last
    # (events between the kernels are not part of the step: they add ~10 us
    # per step of queue work)
    e_start = torch.cuda.Event(enable_timing=True)
    e_end = torch.cuda.Event(enable_timing=True)
    t_wall0 = time.perf_counter()
    e_start.record()
    for _ in range(args.steps):
        for _, fn in parts:
            fn()
    e_end.record()
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t_wall0
    step_ms = e_start.elapsed_time(e_end) / args.steps
    # then K more steps with an event between every two kernels, on the
    # stream they run on, for each kernel's average duration
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(parts) + 1)] for _ in range(args.steps)]
    for e in evs:
        e[0].record()
        for i, (_, fn) in enumerate(parts):
            fn()
            e[i + 1].record()
    torch.cuda.synchronize()
    sclk.__exit__(None, None, None)
    part_all = [[e[i].elapsed_time(e[i + 1]) for e in evs] for i in range(len(parts))]
    part_ms = [sum(x) / args.steps for x in part_all]

    # counted FLOPs (the configs' convention) and each kernel's own algorithmic
    # work per (query, key) pair: forward 4d; dQ kernel 6d (S, dP, dQ; its row
    # terms are O(rows d) beside them); dK/dV kernel 8d (S, dP, dV, dK), with
    # or without the dS stores.  HBM-bound kernels: algorithmic bytes, each
    # input read once and each output written once -- the prep kernel reads O
    # and dO (bf16) and LSE, writes D and LSE log2(e); the dQ-from-dS kernel
    # reads the dS tiles of its blocks (2 bytes per (query, key) pair of the
    # 128 x 64 tiles it visits) and K, writes dQ
    pairs = w.flops("fwd") / (4 * d)
    f_fwd = w.flops("fwd")
    f_bwd = w.flops("bwd") if do_bwd else 0.0
    value = (f_fwd + f_bwd) / (step_ms * 1e-3) / 1e12
    rows = B * H * Sq
    n_kt = -(-Sk // 64)
    ds_tiles = sum(min(n_kt, 2 * (qb + 1)) if w.causal else n_kt for qb in range(-(-Sq // 128)))
    work = {"fwd_kernel": ("mfma", 4 * d * pairs), "bwd_dq_kernel": ("mfma", 6 * d * pairs),
            "bwd_dkdv_kernel": ("mfma", 8 * d * pairs), "bwd_dkdv_kernel_ds": ("mfma", 8 * d * pairs),
            "bwd_prep_kernel": ("hbm", rows * (2 * d * 2 + 4 + 8)),
            "bwd_dq_ds_kernel": ("hbm", B * H * ds_tiles * 128 * 64 * 2 + B * H * Sk * d * 2 + rows * d * 2)}
    kernels = {}
    for i, ((name, _), ms) in enumerate(zip(parts, part_ms)):
        bound, amount = work[name]
        rate = amount / (ms * 1e-3) / (1e12 if bound == "mfma" else 1e9)
        peak = PEAK_BF16_TFLOPS if bound == "mfma" else PEAK_HBM_GBS
        xs = sorted(part_all[i])
        kernels[name] = {"ms": round(ms, 5), "ms_median": round(xs[len(xs) // 2], 5), "ms_min": round(xs[0], 5),
                         "ms_max": round(xs[-1], 5), "bound": bound, "achieved": round(rate, 2),
                         "unit": "TFLOP/s" if bound == "mfma" else "GB/s", "frac": round(rate / peak, 4)}
    dom = max(kernels, key=lambda n: kernels[n]["ms"])
    kd = kernels[dom]
    traffic = read_traffic(dom, w.name)
    roof = {"bound": kd["bound"], "kernel": dom, "achieved": kd["achieved"],
            "peak": PEAK_BF16_TFLOPS if kd["bound"] == "mfma" else PEAK_HBM_GBS, "unit": kd["unit"],
            "frac": kd["frac"], "traffic": traffic, "work_per_launch": work[dom][1],
            "avg_launch_ms": kd["ms"]}

    extra = {}
    if not args.no_extra:
        from workloads import EXTRA_WORKLOADS
        for wid in (2, 3, 4, 6):
            ww = WORKLOADS[wid] if wid in WORKLOADS else EXTRA_WORKLOADS[wid]
            del_ins = [t.to(dev) for t in workload_inputs(ww)]
            qq, kk, vv = del_ins[:3]
            oo = torch.empty_like(qq)
            ll = torch.empty(qq.shape[:3], dtype=torch.float32, device=dev)
            for emu in ww.emu_fracs:
                ms = time_calls(lambda: fa.fa_fwd(qq, kk, vv, oo, ll, causal=ww.causal, scale=ww.scale,
                                                  tau=args.tau, emu_frac=emu), max(10, args.steps), 3,
                                args.warm_seconds / 3)
                tf = ww.flops("fwd") / (ms * 1e-3) / 1e12
                extra[f"{ww.name}" + (f"-emu{emu:g}" if len(ww.emu_fracs) > 1 else "")] = {
                    "ms": round(ms, 5), "tflops": round(tf, 2), "pct_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
                    "emu_realised": round(fa.fa_fwd_realised_emu_frac(ww.d, emu), 4)}
            if wid in (3, 6):
                # the same workload on e4m3 inputs (per-tensor descales), priced
                # against the fp8 MFMA peak
                from workloads import quantise_e4m3
                (q8, qs), (k8, ks), (v8, vs) = (quantise_e4m3(t.cpu()) for t in (qq, kk, vv))
                q8, k8, v8 = q8.to(dev), k8.to(dev), v8.to(dev)
                ms = time_calls(lambda: fa.fa_fwd_fp8(q8, k8, v8, oo, ll, qs, ks, vs, causal=ww.causal,
                                                      scale=ww.scale, tau=args.tau),
                                max(10, args.steps), 3, args.warm_seconds / 3)
                tf = ww.flops("fwd") / (ms * 1e-3) / 1e12
                extra[f"{ww.name}-fp8"] = {
                    "ms": round(ms, 5), "tflops": round(tf, 2), "dtype": "e4m3",
                    "pct_peak_fp8": round(100 * tf / PEAK_FP8_TFLOPS, 2), "peak_tflops": PEAK_FP8_TFLOPS}
                if wid == 3:
                    # ablation of the conditional rescale where the softmax's VALU
                    # work is the bound: tau = 0 corrects on every rise of a row max
                    ms = time_calls(lambda: fa.fa_fwd_fp8(q8, k8, v8, oo, ll, qs, ks, vs, causal=ww.causal,
                                                          scale=ww.scale, tau=0.0),
                                    max(10, args.steps), 3, args.warm_seconds / 3)
                    tf = ww.flops("fwd") / (ms * 1e-3) / 1e12
                    extra[f"{ww.name}-fp8-tau0"] = {
                        "ms": round(ms, 5), "tflops": round(tf, 2), "dtype": "e4m3", "tau": 0.0,
                        "pct_peak_fp8": round(100 * tf / PEAK_FP8_TFLOPS, 2), "peak_tflops": PEAK_FP8_TFLOPS}
                # the same tensors with one factor per 128-row block of Q, K, V
                from workloads import quantise_e4m3_blocks
                (qb8, qbf), (kb8, kbf), (vb8, vbf) = (quantise_e4m3_blocks(t.cpu()) for t in (qq, kk, vv))
                qb8, kb8, vb8, qbf, kbf, vbf = (t.to(dev) for t in (qb8, kb8, vb8, qbf, kbf, vbf))
                ms = time_calls(lambda: fa.fa_fwd_fp8_blocks(qb8, kb8, vb8, qbf, kbf, vbf, oo, ll, causal=ww.causal,
                                                             scale=ww.scale, tau=args.tau),
                                max(10, args.steps), 3, args.warm_seconds / 3)
                tf = ww.flops("fwd") / (ms * 1e-3) / 1e12
                extra[f"{ww.name}-fp8-blocks"] = {
                    "ms": round(ms, 5), "tflops": round(tf, 2), "dtype": "e4m3, one factor per 128-row block",
                    "pct_peak_fp8": round(100 * tf / PEAK_FP8_TFLOPS, 2), "peak_tflops": PEAK_FP8_TFLOPS}
                del qb8, kb8, vb8, qbf, kbf, vbf
                # MXFP4 Q and K (E8M0 scales per 32 dims), e4m3 V: S on the
                # scaled fp4 products, P V in e4m3
                from workloads import quantise_mxfp4
                q4, q4s = (t.to(dev) for t in quantise_mxfp4(qq.cpu()))
                k4, k4s = (t.to(dev) for t in quantise_mxfp4(kk.cpu()))
                ms = time_calls(lambda: fa.fa_fwd_mxfp4(q4, q4s, k4, k4s, v8, oo, ll, vs, causal=ww.causal,
                                                        scale=ww.scale, tau=args.tau),
                                max(10, args.steps), 3, args.warm_seconds / 3)
                tf = ww.flops("fwd") / (ms * 1e-3) / 1e12
                extra[f"{ww.name}-mxfp4"] = {
                    "ms": round(ms, 5), "tflops": round(tf, 2), "dtype": "mxfp4 q,k / e4m3 v,p",
                    "pct_peak_mix": round(100 * tf / PEAK_MXFP4_MIX_TFLOPS, 2),
                    "peak_tflops": round(PEAK_MXFP4_MIX_TFLOPS, 1),
                    "pct_peak_fp8": round(100 * tf / PEAK_FP8_TFLOPS, 2)}
                del q8, k8, v8, q4, q4s, k4, k4s
            if wid == 3:
                # the graded forward's own roofline: algorithmic 4 d FLOPs per
                # counted (query, key) pair over its event-timed launch
                ms3 = extra[ww.name]["ms"]
                work3 = ww.flops("fwd")
                ach = work3 / (ms3 * 1e-3) / 1e12
                extra[f"{ww.name}-roofline"] = {
                    "bound": "mfma", "kernel": "fwd_kernel", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                    "traffic": read_traffic("fwd_kernel", ww.name), "work_per_launch": work3,
                    "avg_launch_ms": ms3}
            if wid in (3, 4):
                # the conditional rescale observed: wavefront-level corrections
                # after each wavefront's first tile (instrumented forward), at
                # tau = 8 and at tau = 0 (every rise of a wavefront's max)
                ev = torch.zeros((ww.B, ww.H, -(-ww.Sq // 32)), dtype=torch.int32, device=dev)
                counts = {}
                for tau_c in (8.0, 0.0):
                    ev.zero_()
                    fa.fa_fwd_rescale_count(qq, kk, vv, oo, ll, ev, causal=ww.causal, scale=ww.scale, tau=tau_c)
                    torch.cuda.synchronize()
                    counts[f"tau{tau_c:g}"] = int(ev.sum().item())
                    # wavefronts by their number of corrections: 0, 1, 2, ... (last bin: 7 or more)
                    hist = torch.bincount(ev.flatten().clamp(max=7).long(), minlength=8)
                    counts[f"tau{tau_c:g}_wavefront_histogram"] = hist.cpu().tolist()
                # (wavefront, tile) steps after the first: each 32-row wavefront
                # visits ceil(visible keys / 128) tiles of 128 keys
                import math as _m
                steps = 0
                for w0 in range(0, ww.Sq, 32):
                    last = min(ww.Sk, w0 + 32) if ww.causal else ww.Sk
                    steps += _m.ceil(last / 128) - 1
                counts["wave_tile_steps_after_first"] = steps * ww.B * ww.H
                extra[f"{ww.name}-rescale_events"] = counts
            if wid == 4:
                # the d = 64 rescale-stress workload on e4m3 inputs (per-tensor factors)
                from workloads import quantise_e4m3
                (q8, qs), (k8, ks), (v8, vs) = (quantise_e4m3(t.cpu()) for t in (qq, kk, vv))
                q8, k8, v8 = q8.to(dev), k8.to(dev), v8.to(dev)
                ms = time_calls(lambda: fa.fa_fwd_fp8(q8, k8, v8, oo, ll, qs, ks, vs, causal=ww.causal,
                                                      scale=ww.scale, tau=args.tau),
                                max(10, args.steps), 3, args.warm_seconds / 3)
                tf = ww.flops("fwd") / (ms * 1e-3) / 1e12
                extra[f"{ww.name}-fp8"] = {
                    "ms": round(ms, 5), "tflops": round(tf, 2), "dtype": "e4m3",
                    "pct_peak_fp8": round(100 * tf / PEAK_FP8_TFLOPS, 2), "peak_tflops": PEAK_FP8_TFLOPS}
                del q8, k8, v8
                # ablation of the conditional rescale: tau = 0 corrects the
                # output on every increase of a row max (the eager online softmax)
                ms = time_calls(lambda: fa.fa_fwd(qq, kk, vv, oo, ll, causal=ww.causal, scale=ww.scale,
                                                  tau=0.0, emu_frac=0.0), max(10, args.steps), 3,
                                args.warm_seconds / 3)
                tf = ww.flops("fwd") / (ms * 1e-3) / 1e12
                extra[f"{ww.name}-emu0-tau0"] = {
                    "ms": round(ms, 5), "tflops": round(tf, 2), "pct_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
                    "emu_realised": 0.0, "tau": 0.0}
            del del_ins, qq, kk, vv, oo, ll

        # split-KV: the causal S=8192 workload as 4 key ranges (fa_fwd_partial
        # into float32 parts) plus fa_merge; the merge is HBM-bound
        ww = WORKLOADS[3]
        qq, kk, vv = [t.to(dev) for t in workload_inputs(ww)][:3]
        n_parts = 4
        bounds = [ww.Sk * i // n_parts for i in range(n_parts + 1)]
        op = torch.empty((n_parts,) + tuple(qq.shape), dtype=torch.float32, device=dev)
        lp = torch.empty((n_parts,) + tuple(qq.shape[:3]), dtype=torch.float32, device=dev)
        om = torch.empty_like(qq)
        lm = torch.empty(qq.shape[:3], dtype=torch.float32, device=dev)

        def partials():
            for i in range(n_parts):
                fa.fa_fwd_partial(qq, kk, vv, op[i], lp[i], 0, bounds[i], bounds[i + 1], causal=True,
                                  scale=ww.scale, tau=args.tau)

        ms_p = time_calls(partials, max(10, args.steps), 3, args.warm_seconds / 3)
        ms_m = time_calls(lambda: fa.fa_merge(op, lp, om, lm), max(10, args.steps), 3, args.warm_seconds / 3)
        rows = ww.B * ww.H * ww.Sq
        merge_bytes = n_parts * rows * (ww.d * 4 + 4) + rows * (ww.d * 2 + 4)
        gbs = merge_bytes / (ms_m * 1e-3) / 1e9
        extra["split_kv"] = {
            "workload": f"{ww.name} as {n_parts} key ranges + merge",
            "partials_ms": round(ms_p, 5), "merge_ms": round(ms_m, 5),
            "tflops": round(ww.flops("fwd") / ((ms_p + ms_m) * 1e-3) / 1e12, 2),
            "merge_roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                               "frac": round(gbs / PEAK_HBM_GBS, 4), "bytes_per_launch": merge_bytes}}
        del qq, kk, vv, op, lp, om, lm

    if do_bwd and not args.no_extra:
        # both backward forms as whole calls, each in both modes: the
        # deterministic flag selects the same kernels (every output element is
        # written once by one workgroup in a fixed order)
        det_ab = {}
        for form, fn in (("ds", bwd_ds), ("split", bwd_split)):
            for det in (0, 1):
                det_ab[f"{form}_deterministic{det}_bwd_ms"] = round(time_calls(
                    lambda: fn(det), max(10, args.steps), 3, args.warm_seconds / 3), 5)
        extra["bwd_forms_and_deterministic_ab"] = det_ab

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_seconds)

    out = {
        "metric": "attention fwd/bwd TFLOP/s and % of MI355X bf16 MFMA peak (1 GPU)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warm_seconds": args.warm_seconds,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16, workloads.py)",
        "config": {"workload": w.name + ("" if do_bwd else " (forward only)"), "B": B, "H": H, "Sq": Sq,
                   "Sk": Sk, "d": d, "causal": w.causal, "tau": args.tau, "emu_frac": args.emu,
                   "deterministic_bwd": bool(args.deterministic),
                   "step": ("fa_fwd + " + ("fa_bwd_ds" if args.bwd == "ds" else "fa_bwd")) if do_bwd
                   else "fa_fwd"},
        "pct_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "peak_tflops": PEAK_BF16_TFLOPS,
        "roofline": roof,
        "cpu_baseline": cpu,
        "gpu_over_cpu_oracle": round(value / cpu["value"], 1) if cpu and cpu.get("value") else None,
        "sclk_observed": sclk.summary(),
        "kernels": kernels,
        "workloads_fwd": extra,
        "wall_s_timed": round(wall_s, 4),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of the emulated-peer AllReduce on one MI355X.

One step = one mscl_allreduce call (algorithm chosen by size: two-shot at
this size — reduce-scatter, signal/wait barrier, all-gather put) over R = 8
emulated ranks of 128 MiB bf16 buffers each (8192 tokens x 8192 hidden,
N(0, 0.5)), inputs already resident in HBM.  Prints ONE JSON line:

  value          algbw = S / t  (S = bytes per rank buffer, t = time per step)
  pct_hbm_peak   (2*R*S / t) / 8 TB/s  -- R*S read plus R*S written
  roofline       the two-shot kernel: algorithmic bytes 2*R*S per launch over
                 its mean launch duration from HIP events on the launch stream;
                 `traffic` from the committed rocprofv3 counter summary
  cpu_baseline   the plain-C oracle on the host cores, on a bounded sample
  latency        p50 of per-call time at 16 KiB (R=8 bf16; R=4 fp32) and the
                 512 KiB decode-shaped case, by HIP events around each call
                 (host launch cost included) and as device time per call
                 replayed from a graph

Options: --gpus N (only 1: the emulation runs on one GPU), --steps K,
--warmup W, --no-cpu-baseline, --sweep (per-size tables to stderr: R=8 bf16
1 KiB..128 MiB and the R=8 fp16 uniform[-1,1] workload 1 KiB..256 MiB, every
algorithm), --main-only (profiler runs), --copy-calibration (also run a
plain 1 GiB device copy, for counter scaling).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "AllReduce algbw GB/s + % of HBM peak, R=8 bf16, 512KB–128MB; p50 µs at 16KB"
HBM_PEAK_GBPS = 8000.0
PMC_SUMMARY = os.path.join(ROOT, "profiles", "twoshot_bf16_r8_128MiB_pmc.md")
# The device code and the host planner that decides what one launch covers
# (algorithm, slices): the committed counter summary is valid only for these.
KERNEL_SOURCES = [os.path.join(ROOT, "allreduce_emulated_peer_amd", "csrc", f)
                  for f in ("kernels.hpp", "channel.hpp", "codec.hpp", "port.hpp", "mscl.hip")]


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def committed_traffic():
    """HBM bytes per launch from the committed counter summary, or None when
    the summary is missing or was taken on different kernel sources."""
    if not os.path.exists(PMC_SUMMARY):
        return None
    text = open(PMC_SUMMARY).read()
    m = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", text)
    t = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != kernel_source_hash():
        return None
    return float(t.group(1))


def oracle_record() -> int:
    """The oracle timed once per workload at its full size, for the record:
    the NumPy oracle on one core and the plain-C oracle on up to 16 threads,
    with the same algbw accounting (S / t)."""
    from allreduce_emulated_peer_amd import workloads as W
    from oracle import allreduce as O
    from oracle import cpu as C

    cores = min(os.cpu_count() or 1, 16)
    rows = []
    for w in (W.integer_small(), W.decode_bf16(), W.prefill_bf16(), W.sweep_fp16(25), W.ragged_outliers_bf16()):
        xs = W.generate_all(w)
        O.allreduce(xs, w.dtype)  # warm: the first pass pays the inputs' first-touch page faults
        t1 = time.perf_counter()
        O.allreduce(xs, w.dtype)
        t_np = time.perf_counter() - t1
        C.allreduce(xs, w.dtype, nthreads=cores)  # warm
        t1 = time.perf_counter()
        C.allreduce(xs, w.dtype, nthreads=cores)
        t_c = time.perf_counter() - t1
        rows.append({"workload": w.name, "numpy_s": round(t_np, 4), "numpy_algbw_GBps": round(w.bytes_per_rank / t_np / 1e9, 3),
                     "c_s": round(t_c, 4), "c_algbw_GBps": round(w.bytes_per_rank / t_c / 1e9, 3)})
        log(f"[oracle-record] {rows[-1]}")
        del xs
    print(json.dumps({"oracle_record": rows, "c_threads": cores, "cpu_count": os.cpu_count()}), flush=True)
    return 0


def profile_legs(M, W, device_inputs, caller) -> int:
    """Three untimed calls of every kernel the bench line reports, for
    rocprofv3 counter passes (one kernel per dispatch, so the counters read per
    dispatch are the kernel's own), then three plain 1 GiB device copies whose
    known bytes calibrate the counters."""
    import ctypes

    import torch

    for w in (W.prefill_bf16(), W.ragged_outliers_bf16(), W.sweep_bf16(21), W.decode_bf16()):
        ins = device_inputs(w)
        outs = [torch.empty_like(t) for t in ins]
        c = caller(w, ins, outs)
        for _ in range(3):
            c()
        torch.cuda.synchronize()
        log(f"[profile-legs] {w.name}: 3 calls")
        del ins, outs
        torch.cuda.empty_cache()
    w = W.prefill_bf16()
    R, rc = w.nranks, w.count // w.nranks
    ins = device_inputs(w)
    blocks = [torch.empty(rc, dtype=torch.bfloat16, device="cuda") for _ in range(R)]
    gathered = [torch.empty(w.count, dtype=torch.bfloat16, device="cuda") for _ in range(R)]
    lib = M.load()
    rs_in = (ctypes.c_void_p * R)(*[t.data_ptr() for t in ins])
    rs_out = (ctypes.c_void_p * R)(*[t.data_ptr() for t in blocks])
    ag_out = (ctypes.c_void_p * R)(*[t.data_ptr() for t in gathered])
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for _ in range(3):
        assert lib.mscl_reduce_scatter(rs_in, rs_out, rc, M.BFLOAT16, R, s) == M.SUCCESS
    for _ in range(3):
        assert lib.mscl_allgather(rs_out, ag_out, rc, M.BFLOAT16, R, s) == M.SUCCESS
    torch.cuda.synchronize()
    log("[profile-legs] reduce_scatter and allgather of the prefill buffers: 3 calls each")
    del ins, blocks, gathered
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log("[profile-legs] copy calibration: 3 plain copies of 1 GiB")
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--latency-iters", type=int, default=1000)
    ap.add_argument("--main-only", action="store_true",
                    help="time only the main workload (for profiler runs): no latency, decode or CPU legs")
    ap.add_argument("--profile-legs", action="store_true",
                    help="for counter runs: three untimed calls of each kernel the bench line reports (prefill, "
                         "ragged R=16, the 2 MiB and 512 KiB R=8 calls, ReduceScatter, AllGather) and three 1 GiB "
                         "device copies for counter calibration; prints nothing on stdout")
    ap.add_argument("--oracle-record", action="store_true",
                    help="CPU only: time the NumPy oracle (one core) and the C oracle once per workload at full size")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: the R emulated ranks all live on one GPU, "
              "and this build runs no multi-GPU path", file=sys.stderr)
        return 2
    if args.oracle_record:
        return oracle_record()

    import torch

    from allreduce_emulated_peer_amd import mscl as M
    from allreduce_emulated_peer_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    M.load()  # raises if the HIP library is missing
    dev = torch.cuda.current_device()
    stream = torch.cuda.current_stream()

    def device_inputs(w):
        xs = W.generate_all(w)
        tdt = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
        out = []
        for x in xs:
            t = torch.from_numpy(x.view(np.int16) if w.dtype == "bf16" else x)
            out.append((t.view(torch.bfloat16) if w.dtype == "bf16" else t).to("cuda"))
            assert out[-1].dtype == tdt
        del xs
        return out

    code = {"fp32": M.FLOAT32, "fp16": M.FLOAT16, "bf16": M.BFLOAT16}

    def caller(w, ins, outs, algo=M.ALGO_AUTO, on_stream=None):
        """A zero-argument launcher with the pointer tables prebuilt (the
        per-call host cost is then the library's own, not Python's)."""
        M.channel_create(w.nranks, dev)
        lib = M.load()
        import ctypes
        in_arr = (ctypes.c_void_p * w.nranks)(*[t.data_ptr() for t in ins])
        out_arr = (ctypes.c_void_p * w.nranks)(*[t.data_ptr() for t in outs])
        s = ctypes.c_void_p((on_stream or stream).cuda_stream)
        n, dt, R = w.count, code[w.dtype], w.nranks

        def call():
            st = lib.mscl_allreduce(in_arr, out_arr, n, dt, R, algo, s)
            if st != M.SUCCESS:
                raise M.MsclError(st, "mscl_allreduce", M.last_error_string())
        return call

    def p50_us(call, iters):
        for _ in range(20):
            call()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
        torch.cuda.synchronize()
        for a, b in ev:
            a.record(stream)
            call()
            b.record(stream)
        torch.cuda.synchronize()
        t = np.array([a.elapsed_time(b) * 1000.0 for a, b in ev])
        return float(np.median(t)), float(t.mean()), float(np.percentile(t, 10)), float(np.percentile(t, 90))

    # Timing-only HIP events: created with hipEventDisableSystemFence, which
    # HIP documents for events used only to measure time (no system-scope
    # cache write-back and invalidate on record).  torch's events keep that
    # fence, which adds ~1.6 us to a bracket around one short call.
    import ctypes as _ct
    _hip = _ct.CDLL("libamdhip64.so")
    _hip.hipEventCreateWithFlags.argtypes = [_ct.POINTER(_ct.c_void_p), _ct.c_uint]
    _hip.hipEventRecord.argtypes = [_ct.c_void_p, _ct.c_void_p]
    _hip.hipEventElapsedTime.argtypes = [_ct.POINTER(_ct.c_float), _ct.c_void_p, _ct.c_void_p]
    _hip.hipEventDestroy.argtypes = [_ct.c_void_p]
    HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000

    def bracket_us(call, iters, before=None):
        """Median time between timing-only HIP events recorded just before
        and just after each call (`before`, if given, runs ahead of the
        first event each time)."""
        def make():
            e = _ct.c_void_p()
            if _hip.hipEventCreateWithFlags(_ct.byref(e), HIP_EVENT_DISABLE_SYSTEM_FENCE) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            return e
        for _ in range(20):
            call()
        evs = [(make(), make()) for _ in range(iters)]
        s_ = _ct.c_void_p(stream.cuda_stream)
        torch.cuda.synchronize()
        for a, b in evs:
            if before is not None:
                before()
            _hip.hipEventRecord(a, s_)
            call()
            _hip.hipEventRecord(b, s_)
        torch.cuda.synchronize()
        t = []
        for a, b in evs:
            ms = _ct.c_float()
            if _hip.hipEventElapsedTime(_ct.byref(ms), a, b) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            t.append(ms.value * 1000.0)
            _hip.hipEventDestroy(a)
            _hip.hipEventDestroy(b)
        return float(np.median(t))

    def p50_us_timing_events(call, iters):
        return bracket_us(call, iters)

    def batch_us(call, iters):
        """Mean time per call of `iters` back-to-back eager calls between two
        events (the way collective benchmarks usually report latency: launch
        throughput and device time overlap, the events are paid once)."""
        for _ in range(20):
            call()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(iters):
            call()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1000.0 / iters

    def graph_us(w, ins, outs, algo=M.ALGO_AUTO, reps=100):
        """Device time per call: `reps` calls captured in one HIP graph and
        replayed, so the host launch cost is amortised (median of 5 replays)."""
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            caller(w, ins, outs, algo, on_stream=side)()  # warm-up outside the capture
        stream.wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            c = caller(w, ins, outs, algo, on_stream=torch.cuda.current_stream())
            for _ in range(reps):
                c()
        g.replay()
        torch.cuda.synchronize()
        ts = []
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            g.replay()
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1000.0 / reps)
        del g
        return float(np.median(ts))

    def rotated_graph_us(w, ins, algo=M.ALGO_AUTO, reps=100):
        """Device time per call over K buffer sets rotated call by call, K the
        fewest whose footprint K * 2RS reaches 512 MiB (past the 256 MB
        Infinity Cache and every L2), replayed from one graph ("cold")."""
        K = max(1, -(-(512 << 20) // (2 * w.nranks * w.bytes_per_rank)))
        sets = [(ins, [torch.empty_like(t) for t in ins])]
        sets += [([t.clone() for t in ins], [torch.empty_like(t) for t in ins]) for _ in range(K - 1)]
        for a_, b_ in sets:
            caller(w, a_, b_, algo)()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cap = [caller(w, a_, b_, algo, on_stream=torch.cuda.current_stream()) for a_, b_ in sets]
            for i in range(max(reps, K)):
                cap[i % K]()
        g.replay()
        torch.cuda.synchronize()
        ts = []
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            g.replay()
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1000.0 / max(reps, K))
        del g, sets, cap
        return float(np.median(ts)), K

    CTYPE = {"fp32": "F32", "fp16": "F16", "bf16": "BF16"}
    ALGO_NAME = {1: "one_shot", 2: "two_shot", 3: "two_shot_fused", 4: "two_shot_port", 5: "two_shot_fused_nobarrier",
                 6: "two_shot_pertile"}

    def describe(w, algo=M.ALGO_AUTO, in_place=False):
        """The algorithm, kernel and synchronisation a call of workload `w` runs."""
        p = M.channel_plan(M.channel_create(w.nranks, dev), w.count, code[w.dtype], algo, in_place=in_place)
        c, R = CTYPE[w.dtype], w.nranks
        cached = "true" if p.cached_puts else "false"
        if p.algo == M.ALGO_ONE_SHOT:
            kernel = f"mscl_oneshot<{c}, {R}, {'true' if in_place else 'false'}>"
            sync = "after-reads barrier per batch (in place)" if in_place else "none (one-shot)"
        elif p.algo == M.ALGO_TWO_SHOT:
            kernel = (f"mscl_twoshot_held<{c}, {R}, {'true' if p.tile_interleave else 'false'}, {cached}>"
                      if p.held_tiles else f"mscl_twoshot<{c}, {R}, {cached}>")
            sync = "signal/wait barrier between reduce-scatter and all-gather"
        elif p.algo == M.ALGO_TWO_SHOT_PERTILE:
            kernel = f"mscl_twoshot_pertile<{c}, {R}, {cached}>"
            sync = "per-tile semaphores between reduce-scatter and all-gather (labelled variant)"
        elif p.algo == M.ALGO_TWO_SHOT_FUSED:
            kernel = f"mscl_twoshot_fused<{c}, {R}, {p.threads_per_workgroup}, {cached}, true>"
            sync = "completion barrier after the puts"
        elif p.algo == M.ALGO_TWO_SHOT_FUSED_NOBARRIER:
            kernel = f"mscl_twoshot_fused<{c}, {R}, {p.threads_per_workgroup}, {cached}, false>"
            sync = "none (labelled variant: completion is the kernel's end on the stream)"
        else:
            kernel = f"mscl_twoshot_port<{c}, {R}>"
            sync = "port-channel flush (proxy completion)"
        d = {"algo": ALGO_NAME[p.algo], "kernel": kernel, "sync": sync}
        if p.slices > 1:
            d["slices"] = p.slices
        return d

    if args.profile_legs:
        return profile_legs(M, W, device_inputs, caller)

    # ---------------------------------------------------------------- main
    w = W.prefill_bf16()
    log(f"[bench] generating {w.name}: R={w.nranks} x {w.bytes_per_rank} B")
    main_xs = W.generate_all(w)  # kept on the host for the CPU baseline
    ins = []
    for x in main_xs:
        ins.append(torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to("cuda"))
    outs = [torch.empty_like(t) for t in ins]
    call = caller(w, ins, outs)
    plan = M.channel_plan(M.channel_create(w.nranks, dev), w.count, M.BFLOAT16, M.ALGO_AUTO)
    algo_name = {1: "one_shot", 2: "two_shot", 3: "two_shot_fused"}[plan.algo]
    log(f"[bench] plan: {algo_name}, {plan.workgroups_per_rank} workgroups/rank x {plan.threads_per_workgroup} "
        f"threads, {plan.vectors_per_thread} vectors/thread, {plan.slices} slice(s) of {plan.slice_elems} elements, "
        f"{plan.held_tiles} tiles held in LDS per workgroup")
    launches = plan.slices  # kernel launches per step (one per slice)
    main_kernel = (f"mscl_twoshot_held<BF16, {w.nranks}, {'true' if plan.tile_interleave else 'false'}, "
                   f"{'true' if plan.cached_puts else 'false'}>"
                   if plan.held_tiles else f"mscl_twoshot<BF16, {w.nranks}, false>")
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    # Per-step kernel time from timing-only HIP events (no system-scope cache
    # write-back at each record), on the stream the kernel runs on.
    def timing_event():
        e = _ct.c_void_p()
        if _hip.hipEventCreateWithFlags(_ct.byref(e), HIP_EVENT_DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        return e
    ev = [(timing_event(), timing_event()) for _ in range(args.steps)]
    s_main = _ct.c_void_p(stream.cuda_stream)
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        call()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1000.0 / args.steps
    # The same number of steps again, untimed by the wall clock, each between
    # two timing-only events (kept out of the timed steps above, where their
    # records would sit between the calls).
    for a, b in ev:
        _hip.hipEventRecord(a, s_main)
        call()
        _hip.hipEventRecord(b, s_main)
    torch.cuda.synchronize()
    kern = []
    for a, b in ev:
        ms = _ct.c_float()
        if _hip.hipEventElapsedTime(_ct.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        kern.append(ms.value)
        _hip.hipEventDestroy(a)
        _hip.hipEventDestroy(b)
    kern_ms = np.array(kern)
    S = w.bytes_per_rank
    alg_bytes = w.algorithmic_bytes
    algbw = S / (ms_per_step / 1000.0) / 1e9
    hbm_gbps = alg_bytes / (ms_per_step / 1000.0) / 1e9
    achieved = alg_bytes / (kern_ms.mean() / 1000.0) / 1e9
    log(f"[bench] {ms_per_step:.4f} ms/step wall, kernel mean {kern_ms.mean():.4f} ms (p50 {np.median(kern_ms):.4f}),"
        f" algbw {algbw:.1f} GB/s, {hbm_gbps:.1f} GB/s algorithmic HBM ({100 * hbm_gbps / HBM_PEAK_GBPS:.1f}% of peak)")
    traffic = committed_traffic()
    # One step is `launches` kernel launches of equal size (the slices), timed
    # together between the events: per launch, algorithmic bytes and time are
    # both the step's divided by `launches`, so `achieved` is the same ratio.
    launch_ms = float(kern_ms.mean()) / launches
    roofline = {"bound": "hbm", "kernel": main_kernel, "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": None if traffic is None else int(traffic), "traffic_unit": "bytes per launch",
                "traffic_gbps": None if traffic is None else round(traffic / (launch_ms / 1000.0) / 1e9, 1),
                "algorithmic_bytes_per_launch": alg_bytes // launches, "mean_launch_ms": round(launch_ms, 5),
                "launches_per_step": launches, "mean_step_kernel_ms": round(float(kern_ms.mean()), 5)}
    del ins, outs
    torch.cuda.empty_cache()

    # --------------------------------------------------- latency + decode
    latency, decode = {}, None
    for lw in (() if args.main_only else (W.sweep_bf16(14), W.integer_small())):
        li = device_inputs(lw)
        lo = [torch.empty_like(t) for t in li]
        p50, mean, p10, p90 = p50_us(caller(lw, li, lo), args.latency_iters)
        p50_te = p50_us_timing_events(caller(lw, li, lo), args.latency_iters)
        dev_us = graph_us(lw, li, lo)
        b_us = batch_us(caller(lw, li, lo), args.latency_iters)
        latency[f"p50_us_16KiB_{lw.name}"] = round(p50, 2)
        latency[f"p10_p90_us_16KiB_{lw.name}"] = [round(p10, 2), round(p90, 2)]
        latency[f"p50_us_timing_events_16KiB_{lw.name}"] = round(p50_te, 2)
        latency[f"graph_us_per_call_16KiB_{lw.name}"] = round(dev_us, 2)
        latency[f"batch_us_per_call_16KiB_{lw.name}"] = round(b_us, 2)
        log(f"[bench] {lw.name}: p50 {p50:.2f} us per call (torch events), {p50_te:.2f} us (timing-only events), "
            f"{dev_us:.2f} us per call replayed from a graph, {b_us:.2f} us per call over back-to-back eager calls")
    if latency:
        # latency floor: the smallest event p50 over the R = 8 bf16 sizes up to 64 KiB
        floor = {}
        for k in (10, 12, 14, 16):
            fw = W.sweep_bf16(k)
            fi = device_inputs(fw)
            fo = [torch.empty_like(t) for t in fi]
            floor[fw.bytes_per_rank] = p50_us(caller(fw, fi, fo), args.latency_iters)[0]
            del fi, fo
        best = min(floor, key=floor.get)
        latency["floor_p50_us_le_64KiB_r8_bf16"] = round(floor[best], 2)
        latency["floor_at_bytes"] = best
        latency["note"] = ("p50_us: torch (HIP) events around each call; p50_us_timing_events: HIP events created "
                           "with hipEventDisableSystemFence around each call; graph_us_per_call: 100 calls "
                           "replayed from one graph (device time per call); batch_us_per_call: torch events around "
                           "back-to-back eager calls, divided by their number; floor: smallest torch-event p50 over "
                           "1, 4, 16 and 64 KiB per rank")
    host = None
    if not args.main_only:
        # Host cost of one call (ctypes + validation + launch): CPU clock
        # around each of 10^4 calls at 16 KiB, the stream drained every 100
        # calls so a full queue never makes the host wait on the GPU; and of
        # a call that launches nothing (count = 0), which isolates the launch.
        hw = W.sweep_bf16(14)
        hi_ = device_inputs(hw)
        ho = [torch.empty_like(t) for t in hi_]
        c16 = caller(hw, hi_, ho)
        import dataclasses
        c0 = caller(dataclasses.replace(hw, count=0), hi_, ho)
        for c in (c16, c0):
            for _ in range(100):
                c()
        torch.cuda.synchronize()
        res = {}
        clock = time.perf_counter
        for name, c in (("with_launch", c16), ("no_launch_count0", c0)):
            per = np.empty(10000)
            for b in range(100):
                for i in range(100):
                    t1 = clock()
                    c()
                    per[b * 100 + i] = clock() - t1
                torch.cuda.synchronize()
            res[name] = (float(np.median(per)) * 1e6, float(per.mean()) * 1e6)
        host = {"us_per_call": round(res["with_launch"][0], 2), "us_per_call_mean": round(res["with_launch"][1], 2),
                "us_per_call_count0": round(res["no_launch_count0"][0], 2),
                "note": "CPU clock around each of 10^4 calls from Python (ctypes), 16 KiB R=8 bf16 on torch's "
                        "current stream, drained every 100 calls; median (and mean)"}
        log(f"[bench] host cost: median {host['us_per_call']} us per call (mean {host['us_per_call_mean']}), "
            f"{host['us_per_call_count0']} us with count = 0")
        del hi_, ho

    if not args.main_only:
        dw = W.decode_bf16()
        di = device_inputs(dw)
        do = [torch.empty_like(t) for t in di]
        p50, mean, p10, p90 = p50_us(caller(dw, di, do), args.latency_iters)
        dev_us = graph_us(dw, di, do)
        # Cold: rotate K buffer sets whose total footprint (K * 2RS = 512 MiB)
        # exceeds the 256 MB Infinity Cache, so every call starts from HBM.
        K = -(-(512 << 20) // (2 * dw.nranks * dw.bytes_per_rank))
        sets = [(di, do)] + [([t.clone() for t in di], [torch.empty_like(t) for t in di]) for _ in range(K - 1)]
        calls = [caller(dw, a, b) for a, b in sets]
        for c in calls:
            c()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(4 * K)]
        for i, (a, b) in enumerate(ev):
            a.record(stream)
            calls[i % K]()
            b.record(stream)
        torch.cuda.synchronize()
        cold_p50 = float(np.median([a.elapsed_time(b) * 1000.0 for a, b in ev]))
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cap = [caller(dw, a, b, on_stream=torch.cuda.current_stream()) for a, b in sets]
            for _ in range(2):
                for c in cap:
                    c()
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        cold_dev = a.elapsed_time(b) * 1000.0 / (2 * K)
        del g, sets, calls, cap
        p50_te = p50_us_timing_events(caller(dw, di, do), args.latency_iters)
        nob_us = graph_us(dw, di, do, M.ALGO_TWO_SHOT_FUSED_NOBARRIER)
        decode = {"workload": dw.name, **describe(dw),
                  "nobarrier_variant_graph_us_per_call": round(nob_us, 2),
                  "hot": {"p50_us": round(p50, 2), "p10_p90_us": [round(p10, 2), round(p90, 2)],
                          "p50_us_timing_events": round(p50_te, 2),
                          "graph_us_per_call": round(dev_us, 2),
                          "algbw_GBps_graph": round(dw.bytes_per_rank / dev_us / 1e3, 1),
                          "pct_hbm_peak_graph": round(100 * dw.algorithmic_bytes / dev_us / 1e3 / HBM_PEAK_GBPS, 1),
                          "cache": "same buffers every call (8 MiB footprint stays in cache)"},
                  "cold": {"p50_us": round(cold_p50, 2), "graph_us_per_call": round(cold_dev, 2),
                           "algbw_GBps_graph": round(dw.bytes_per_rank / cold_dev / 1e3, 1),
                           "pct_hbm_peak_graph": round(100 * dw.algorithmic_bytes / cold_dev / 1e3 / HBM_PEAK_GBPS, 1),
                           "cache": f"{K} buffer sets rotated ({K * 2 * dw.nranks * dw.bytes_per_rank >> 20} MiB footprint)"}}
        log(f"[bench] {dw.name}: hot p50 {p50:.2f} us, graph {dev_us:.2f} us/call; "
            f"cold p50 {cold_p50:.2f} us, graph {cold_dev:.2f} us/call")
        del di, do
        torch.cuda.empty_cache()

    ragged = None
    if not args.main_only:
        rw = W.ragged_outliers_bf16()
        ri = device_inputs(rw)
        ro = [torch.empty_like(t) for t in ri]
        rplan = M.channel_plan(M.channel_create(rw.nranks, dev), rw.count, M.BFLOAT16, M.ALGO_AUTO)
        t_r = graph_us(rw, ri, ro, M.ALGO_AUTO, reps=10)
        ragged = {"workload": rw.name, **describe(rw), "us": round(t_r, 1), "algbw_GBps": round(rw.bytes_per_rank / t_r / 1e3, 1),
                  "pct_hbm_peak": round(100 * rw.algorithmic_bytes / t_r / 1e3 / HBM_PEAK_GBPS, 1)}
        log(f"[bench] {rw.name}: {t_r:.1f} us, {ragged['pct_hbm_peak']}% of HBM peak")
        del ri, ro
        torch.cuda.empty_cache()

    size_curve = None
    if not args.main_only:
        # The metric's size range, R = 8 bf16 from 512 KiB to 128 MiB per rank,
        # with AUTO's pick: device time per call replayed from a graph, over the
        # same buffers every call ("hot") and over buffer sets rotated past the
        # Infinity Cache ("cold").  Below 32 MiB per rank the hot call's 2RS
        # footprint fits the 256 MB Infinity Cache, so its HBM percentage
        # measures cache bandwidth; the cold figure is the HBM one.
        size_curve = {"note": "R=8 bf16, AUTO's pick; us per call from graph replay: hot = same buffers every call, "
                              "cold = buffer sets rotated so that the replayed footprint reaches 512 MiB (K sets); "
                              "pct_hbm_peak = 2RS/t over 8 TB/s; cache_resident: the hot call's 2RS fits the 256 MB "
                              "Infinity Cache, so only its cold figure measures HBM; *_variant_hot_us: labelled "
                              "variants AUTO never picks (fused without its barrier, per-tile semaphores)"}
        for k in range(19, 28):
            cw = W.sweep_bf16(k)
            ci_ = device_inputs(cw)
            co_ = [torch.empty_like(t) for t in ci_]
            reps = 50 if cw.bytes_per_rank <= (4 << 20) else 5
            t_h = graph_us(cw, ci_, co_, M.ALGO_AUTO, reps)
            t_c, K = rotated_graph_us(cw, ci_, M.ALGO_AUTO, reps)
            entry = describe(cw)
            entry.update({
                "hot_us": round(t_h, 2), "cold_us": round(t_c, 2), "cold_sets": K,
                "algbw_GBps_hot": round(cw.bytes_per_rank / t_h / 1e3, 1),
                "algbw_GBps_cold": round(cw.bytes_per_rank / t_c / 1e3, 1),
                "pct_hbm_peak_hot": round(100 * cw.algorithmic_bytes / t_h / 1e3 / HBM_PEAK_GBPS, 1),
                "pct_hbm_peak_cold": round(100 * cw.algorithmic_bytes / t_c / 1e3 / HBM_PEAK_GBPS, 1),
                "cache_resident": cw.algorithmic_bytes <= (256 << 20)})
            if entry["algo"] == "two_shot_fused":
                entry["nobarrier_variant_hot_us"] = round(
                    graph_us(cw, ci_, co_, M.ALGO_TWO_SHOT_FUSED_NOBARRIER, reps), 2)
            if k in (19, 22, 26):  # the per-tile-semaphore variant beside AUTO's pick (hot)
                entry["pertile_variant_hot_us"] = round(graph_us(cw, ci_, co_, M.ALGO_TWO_SHOT_PERTILE, reps), 2)
            size_curve[f"{cw.bytes_per_rank}B"] = entry
            del ci_, co_
            torch.cuda.empty_cache()
        log(f"[bench] size curve (hot/cold GB/s): " + ", ".join(
            f"{k} {v['algbw_GBps_hot']}/{v['algbw_GBps_cold']} ({v['algo']})" for k, v in size_curve.items()
            if k != "note"))

    fp16_sweep = None
    if not args.main_only:
        # The fp16 uniform[-1, 1] workload at R = 8, 1 KiB .. 256 MiB per rank:
        # every algorithm's device time (graph replay, same buffers), AUTO's
        # pick, and the crossovers.  Inputs are drawn on the device (seeded
        # torch generator, uniform[-1, 1] in binary32 rounded to fp16): timing
        # does not depend on the values, and host generation of 2 GiB would
        # dominate the run.
        fp16_sweep = {"note": "R=8 fp16 uniform[-1,1] (drawn on the device), bytes per rank 2^k; us per call from "
                              "graph replay over the same buffers (hot: up to 16 MiB per rank the 2RS footprint "
                              "fits the Infinity Cache); auto = AUTO's pick; crossovers: smallest size at which "
                              "the next algorithm is faster", "points": {}}
        gen = torch.Generator(device="cuda")
        prev_best = None
        cross = {}
        for k in range(10, 29):
            sw = W.sweep_fp16(k)
            gen.manual_seed(20261202 + k)
            si = [(torch.rand(sw.count, generator=gen, device="cuda") * 2 - 1).to(torch.float16)
                  for _ in range(sw.nranks)]
            so = [torch.empty_like(t) for t in si]
            reps = 50 if sw.bytes_per_rank <= (4 << 20) else 5
            t = {name: graph_us(sw, si, so, a, reps) for a, name in
                 ((M.ALGO_ONE_SHOT, "one_shot"), (M.ALGO_TWO_SHOT, "two_shot"), (M.ALGO_TWO_SHOT_FUSED, "two_shot_fused"))}
            d = describe(sw)
            t_auto = t[d["algo"]]
            best = min(t, key=t.get)
            if prev_best is not None and best != prev_best and f"{prev_best}->{best}" not in cross:
                cross[f"{prev_best}->{best}"] = sw.bytes_per_rank
            prev_best = best
            fp16_sweep["points"][str(sw.bytes_per_rank)] = {
                "auto": d["algo"], "kernel": d["kernel"], "us": round(t_auto, 2),
                "algbw_GBps": round(sw.bytes_per_rank / t_auto / 1e3, 1),
                "pct_hbm_peak": round(100 * sw.algorithmic_bytes / t_auto / 1e3 / HBM_PEAK_GBPS, 1),
                "one_shot_us": round(t["one_shot"], 2), "two_shot_us": round(t["two_shot"], 2),
                "fused_us": round(t["two_shot_fused"], 2)}
            del si, so
            torch.cuda.empty_cache()
        fp16_sweep["crossovers_bytes_per_rank"] = cross
        fp16_sweep["p50_16KiB_graph_us"] = fp16_sweep["points"][str(16 << 10)]["us"]
        log(f"[bench] fp16 sweep crossovers: {cross}")

    pipeline = None
    if not args.main_only:
        # Tensor-parallel use: a producer kernel writes the inputs just before
        # the call (the row-parallel GEMM's partial sums) and a consumer kernel
        # reads the outputs just after it (the next layer).  Producer = copy from
        # a source set into the inputs, consumer = copy from the outputs into a
        # sink set, all replayed from one graph; the call's share of the time is
        # (producer + call + consumer) - (producer + consumer), so it includes
        # what the call's put policy saves or costs its neighbours.
        pipeline = {"note": "R=8 bf16, AUTO's pick; us per iteration of producer (copy into the inputs), call, "
                            "consumer (copy out of the outputs), replayed from one graph, 16 iterations, median of "
                            "5 replays; allreduce_share_us = with_allreduce_us - producer_consumer_us"}
        for k in (19, 22, 23, 24):  # 512 KiB, 4, 8 and 16 MiB per rank
            pw = W.sweep_bf16(k)
            src = device_inputs(pw)
            pin = [torch.empty_like(t) for t in src]
            pout = [torch.empty_like(t) for t in src]
            sink = [torch.empty_like(t) for t in src]
            reps = 16

            def produce():
                for a_, b_ in zip(pin, src):
                    a_.copy_(b_)

            def consume():
                for a_, b_ in zip(sink, pout):
                    a_.copy_(b_)

            produce()
            caller(pw, pin, pout)()
            consume()
            torch.cuda.synchronize()
            res = {}
            for with_call in (False, True):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    c = caller(pw, pin, pout, M.ALGO_AUTO, on_stream=torch.cuda.current_stream())
                    for _ in range(reps):
                        produce()
                        if with_call:
                            c()
                        consume()
                g.replay()
                torch.cuda.synchronize()
                ts = []
                for _ in range(5):
                    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    a.record(stream)
                    g.replay()
                    b.record(stream)
                    torch.cuda.synchronize()
                    ts.append(a.elapsed_time(b) * 1000.0 / reps)
                res[with_call] = float(np.median(ts))
                del g
            pplan = M.channel_plan(M.channel_create(pw.nranks, dev), pw.count, M.BFLOAT16, M.ALGO_AUTO)
            pipeline[f"{pw.bytes_per_rank}B"] = {
                "algo": {1: "one_shot", 2: "two_shot", 3: "two_shot_fused"}[pplan.algo],
                "cached_puts": pplan.cached_puts, "producer_consumer_us": round(res[False], 2),
                "with_allreduce_us": round(res[True], 2), "allreduce_share_us": round(res[True] - res[False], 2)}
            del src, pin, pout, sink
            torch.cuda.empty_cache()
        log(f"[bench] between producer and consumer: " + ", ".join(
            f"{k} {v['allreduce_share_us']} us" for k, v in pipeline.items() if k != "note"))

    port = None
    if not args.main_only:
        # The port channel (all-gather puts done by the host proxy on the SDMA
        # engines) against the memory-channel two-shot, R = 8 bf16, device time
        # per call between timing-only events.  The first call on a channel set
        # starts the proxy and the engines; it is timed apart.
        port = {"note": "us per call between timing-only HIP events, R=8 bf16; first_call_ms: proxy and SDMA "
                        "engine start-up, once per channel set"}
        for k in (19, 24, 27):  # 512 KiB, 16 MiB, 128 MiB per rank
            pw = W.sweep_bf16(k)
            pi = device_inputs(pw)
            po = [torch.empty_like(t) for t in pi]
            cp = caller(pw, pi, po, M.ALGO_TWO_SHOT_PORT)
            if "first_call_ms" not in port:
                t1 = time.perf_counter()
                cp()
                torch.cuda.synchronize()
                port["first_call_ms"] = round((time.perf_counter() - t1) * 1000.0, 1)
            iters = 50 if pw.bytes_per_rank <= (16 << 20) else 15
            t_port = bracket_us(cp, iters)
            t_two = bracket_us(caller(pw, pi, po, M.ALGO_TWO_SHOT), iters)
            port[f"{pw.bytes_per_rank}B"] = {"port_us": round(t_port, 1), "two_shot_us": round(t_two, 1),
                                            "port_algbw_GBps": round(pw.bytes_per_rank / t_port / 1e3, 1)}
            log(f"[bench] port channel {pw.bytes_per_rank} B: {t_port:.1f} us (two-shot {t_two:.1f} us)")
            del pi, po
            torch.cuda.empty_cache()

    collectives = None
    if not args.main_only:
        # ReduceScatter of the prefill buffers (16 MiB blocks) and AllGather of
        # the blocks back; algorithmic bytes: everything read once + written once
        import ctypes
        R, rc = w.nranks, w.count // w.nranks
        ci = device_inputs(w)
        blocks = [torch.empty(rc, dtype=torch.bfloat16, device="cuda") for _ in range(R)]
        gathered = [torch.empty(w.count, dtype=torch.bfloat16, device="cuda") for _ in range(R)]
        lib = M.load()
        rs_in = (ctypes.c_void_p * R)(*[t.data_ptr() for t in ci])
        rs_out = (ctypes.c_void_p * R)(*[t.data_ptr() for t in blocks])
        ag_out = (ctypes.c_void_p * R)(*[t.data_ptr() for t in gathered])

        def timed(fn, reps=5):
            g = torch.cuda.CUDAGraph()
            fn(stream.cuda_stream)
            torch.cuda.synchronize()
            with torch.cuda.graph(g):
                for _ in range(reps):
                    fn(torch.cuda.current_stream().cuda_stream)
            g.replay()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            g.replay()
            b.record(stream)
            torch.cuda.synchronize()
            return a.elapsed_time(b) * 1000.0 / reps

        def rs(s):
            assert lib.mscl_reduce_scatter(rs_in, rs_out, rc, M.BFLOAT16, R, ctypes.c_void_p(s)) == M.SUCCESS

        def ag(s):
            assert lib.mscl_allgather(rs_out, ag_out, rc, M.BFLOAT16, R, ctypes.c_void_p(s)) == M.SUCCESS
        t_rs, t_ag = timed(rs), timed(ag)
        b_rs = R * S + R * rc * 2  # R inputs of S read, R blocks written
        b_ag = R * rc * 2 + R * S  # R blocks read, R outputs of S written
        collectives = {
            "reduce_scatter": {"shape": f"R=8 bf16, {S} B inputs, {rc * 2} B blocks", "us": round(t_rs, 1),
                               "GBps": round(b_rs / t_rs / 1e3, 1),
                               "pct_hbm_peak": round(100 * b_rs / t_rs / 1e3 / HBM_PEAK_GBPS, 1)},
            "allgather": {"shape": f"R=8 bf16, {rc * 2} B blocks, {S} B outputs", "us": round(t_ag, 1),
                          "GBps": round(b_ag / t_ag / 1e3, 1),
                          "pct_hbm_peak": round(100 * b_ag / t_ag / 1e3 / HBM_PEAK_GBPS, 1)},
            "note": "device time per call, graph replay; bytes = data read once + written once"}
        log(f"[bench] reduce_scatter {t_rs:.1f} us ({collectives['reduce_scatter']['GBps']} GB/s), "
            f"allgather {t_ag:.1f} us ({collectives['allgather']['GBps']} GB/s)")
        del ci, blocks, gathered
        torch.cuda.empty_cache()

    if args.sweep:
        # Cold calls: a 768 MiB device copy (through the 256 MB Infinity Cache
        # and every L2) runs before each call, and timing-only HIP events
        # bracket the call alone.  The copy takes ~100 us, so the host is always ahead of the
        # GPU and the event interval is the call's device time.  Sizes from
        # 32 MiB per rank up are cold by construction (2RS >= 512 MiB).
        fl_src = torch.empty(768 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        fl_dst = torch.empty_like(fl_src)

        def cold_us(call, iters=15, flush_bytes=None):
            src, dst = (fl_src, fl_dst) if flush_bytes is None else (fl_src[:flush_bytes], fl_dst[:flush_bytes])
            return bracket_us(call, iters, before=lambda: dst.copy_(src))

        algos = ((M.ALGO_ONE_SHOT, "one"), (M.ALGO_TWO_SHOT, "two"), (M.ALGO_TWO_SHOT_FUSED, "fused"))
        cw = W.sweep_bf16(10)
        ci_, co_ = device_inputs(cw), None
        co_ = [torch.empty_like(t) for t in ci_]
        warm = cold_us(caller(cw, ci_, co_, M.ALGO_ONE_SHOT), iters=31, flush_bytes=1 << 20)
        log(f"[bench] cold-method calibration: the 1 KiB one-shot bracketed the same way after a 1 MiB copy "
            f"(its buffers stay cached): {warm:.2f} us; graph replay gives "
            f"{graph_us(cw, ci_, co_, M.ALGO_ONE_SHOT, 50):.2f} us")
        del ci_, co_
        sweeps = (("bf16", W.sweep_bf16, range(10, 28)), ("fp16", W.sweep_fp16, range(10, 29)))
        for tag, make, ks in sweeps:
            log(f"[bench] sweep R=8 {tag}: bytes/rank; hot us one/two/fused (same buffers, graph-replayed device "
                "time); best hot algbw GB/s and % HBM peak; AUTO's pick; cold us one/two/fused (caches flushed "
                "before each call, below 32 MiB)")
            for k in ks:
                sw = make(k)
                si = device_inputs(sw)
                so = [torch.empty_like(t) for t in si]
                reps = 50 if sw.bytes_per_rank <= (4 << 20) else 5
                t = {name: graph_us(sw, si, so, algo, reps) for algo, name in algos}
                best = min(t.values())
                pick = {1: "one", 2: "two", 3: "fused"}[M.select_algo(sw.count, code[sw.dtype], sw.nranks)]
                cold = ""
                if sw.bytes_per_rank < (32 << 20):
                    c = {name: cold_us(caller(sw, si, so, algo)) for algo, name in algos}
                    cold = f"   cold {c['one']:9.2f} {c['two']:9.2f} {c['fused']:9.2f}"
                log(f"[sweep-{tag}] {sw.bytes_per_rank:>10d} {t['one']:9.2f} {t['two']:9.2f} {t['fused']:9.2f} "
                    f"{sw.bytes_per_rank / best / 1e3:8.1f} {100 * sw.algorithmic_bytes / best / 1e3 / HBM_PEAK_GBPS:6.1f}"
                    f" {pick:5s}{cold}")
                del si, so
                torch.cuda.empty_cache()
        del fl_src, fl_dst
        torch.cuda.empty_cache()

    if args.copy_calibration:
        nbytes = 1 << 30
        src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        src.fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: 3 plain copies of {nbytes} bytes")
        del src, dst

    # ---------------------------------------------------------- CPU oracle
    cpu = None
    if not (args.no_cpu_baseline or args.main_only):
        from oracle import cpu as C

        cores = min(os.cpu_count() or 1, 16)
        outs_h = [np.empty(w.count, dtype=np.uint16) for _ in range(w.nranks)]
        C.allreduce(main_xs, "bf16", nthreads=cores, outputs=outs_h)  # warm (first touch of the outputs)
        reps, t_total = 0, 0.0
        while t_total < 15.0 and reps < 60:
            t1 = time.perf_counter()
            C.allreduce(main_xs, "bf16", nthreads=cores, outputs=outs_h)
            t_total += time.perf_counter() - t1
            reps += 1
        t_per = t_total / reps
        cpu = {"value": round(w.bytes_per_rank / t_per / 1e9, 3), "unit": "GB/s", "cores": cores,
               "host_cpu_count": os.cpu_count(), "kind": "oracle",
               "sample": f"plain-C oracle on the whole {w.name} workload (8 x {w.count} bf16 elements, the same "
                         f"inputs as the GPU run), {reps} runs, {t_per * 1000:.1f} ms per run; same algbw "
                         f"accounting (S/t)"}
        del outs_h
        log(f"[bench] cpu oracle: {cpu['value']} GB/s algbw on {cores} threads")

    line = {
        "metric": METRIC, "value": round(algbw, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "nranks": w.nranks, "elements_per_rank": w.count,
                   "bytes_per_rank": S, "accumulate": "f32", "algo": f"auto -> {algo_name}",
                   "workgroups_per_rank": plan.workgroups_per_rank, "slices": plan.slices,
                   "held_tiles_per_workgroup": plan.held_tiles, "parallelism": "8 emulated ranks on 1 GPU"},
        "pct_hbm_peak": round(100 * hbm_gbps / HBM_PEAK_GBPS, 2),
        "hbm_gbps_algorithmic": round(hbm_gbps, 1),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "latency": latency,
        "host_api": host,
        "algbw_512KiB_to_128MiB": size_curve,
        "fp16_sweep_1KiB_to_256MiB": fp16_sweep,
        "decode_512KiB": decode,
        "between_producer_and_consumer": pipeline,
        "ragged_r16": ragged,
        "port_channel": port,
        "collectives": collectives,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

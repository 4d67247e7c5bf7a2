#!/usr/bin/env python3
"""Benchmark of the MoE token routing/dispatch/combine path on one MI355X.

One step = moe_route_topk (or moe_route_topk_grouped with --route-groups) +
moe_dispatch (or moe_dispatch_packed with --layout packed) + moe_combine (or
moe_combine_residual_rmsnorm with --epilogue rmsnorm, or its fp8-output form
moe_combine_residual_rmsnorm_fp8 with --epilogue rmsnorm-fp8), back to back on one
stream, over one batch of seeded synthetic input already resident in HBM.
With plain top-k the first two are the single call moe_route_dispatch (or
moe_route_dispatch_packed; identical outputs; --separate-route calls them
apart).

The headline workload is the largest that fits one GPU: GLM-style prefill
(32768 tokens, hidden 6144, 128 experts, top-8, fp8 dispatch).  W untimed
warm-up steps, then exactly K timed steps between device synchronisations,
with nothing else in the stream: no timing events inside the timed region.
Prints one JSON line (stdout):

  value     tokens/s of the whole job (one GPU), from the host clock around
            the K timed steps
  config    the workload plus effective HBM GB/s and fraction of the 8 TB/s
            peak, from the algorithmic byte model (each row read once and
            written k times, unfilled slots not counted); per-call kernel
            times from a separate timing pass; the copy floors (--floor);
            and, by default, the Mixtral-like and DeepSeek-R1-like prefill
            workloads measured the same way (other_workloads)
  roofline  the dominant kernel (combine): algorithmic bytes per launch over
            its mean launch time, from HIP events recorded on the launch
            stream around every combine call of the timing pass
  roofline_dispatch  the same for the dispatch call (count + pack launches,
            or route + pack for the one-call path)
  cpu_baseline  the CPU oracle on a bounded sample of the same workload, on
            the host's cores (threads over tokens for route, pack and
            combine; slot assignment serial) and on one thread

Consecutive steps cycle through several copies of every buffer (inputs,
outputs and the fixed-slot buffers) so that each step's data was last touched
many steps earlier: the 256 MB last-level cache in front of HBM cannot serve
a small workload's working set from a previous step.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

METRIC = "dispatch+combine tokens/s and effective HBM GB/s (% of peak), 1 MI355X"
EPILOGUE_LABEL = {None: "", "rmsnorm": "+residual+rmsnorm", "rmsnorm-fp8": "+residual+rmsnorm+fp8"}
HBM_PEAK_GBPS = 8000.0
DEFAULT_WORKLOAD = "glm_prefill"
SECONDARY = ["mixtral_prefill", "dsr1_prefill"]
FLOOR_SRC = os.path.join(ROOT, "bench_floor.hip")
FLOOR_LIB = os.path.join(ROOT, "bench_floor.so")


def algorithmic_bytes(w: W.Workload, epilogue: str | None = None) -> dict:
    """Bytes each step must move: every row read once and written k times.
    With the fused residual + RMSNorm epilogue ("rmsnorm"), combine also
    reads the residual and gamma and writes the updated residual (its
    normalised rows take the place of the plain output); "rmsnorm-fp8"
    writes the normalised rows as E4M3 codes + per-128 fp32 scales instead."""
    T, H, E, k = w.T, w.H, w.E, w.k
    row = (H + H // 32) if w.fp8 else 2 * H
    out_row = (H + H // 32) if epilogue == "rmsnorm-fp8" else 2 * H
    b = {
        "route": T * E * 4 + T * k * 8,
        "count_scan_slot": T * k * 12 + E * 4,
        "pack": T * H * 2 + T * k * 4 + T * k * row,
        "combine": T * k * 2 * H + T * k * 8 + T * out_row + ((T * H * 4 + H * 2) if epilogue else 0),
    }
    b["total"] = sum(b.values())
    return b


def combine_source_hash() -> str:
    """Hash of the combine kernel's sources, to tell whether a committed
    counter measurement still describes the kernel that runs."""
    import hashlib
    h = hashlib.sha256()
    for f in ("combine.hip", "device_common.hpp"):
        with open(os.path.join(ROOT, "combine_moe_route_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(w: W.Workload):
    """HBM bytes per combine launch from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, copy-calibrated), or None when there is
    none for this workload or the kernel changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{w.name}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and line.startswith("combine-"):
            key, val = line.split(":", 1)
            fields[key.strip()] = val.strip()
    if fields.get("combine-source-sha256-16") != combine_source_hash():
        return None
    try:
        return int(fields["combine-traffic-bytes-per-launch"])
    except (KeyError, ValueError):
        return None


def host_cpu() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_threads() -> int:
    """Threads for the host-cores baseline: the cores this process may run
    on, at most 16 (a one-GPU share of the machine's host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _balanced_expert_ranges(filled, parts: int):
    """Split experts into at most `parts` consecutive ranges with about the
    same number of filled rows each; returns (e0, e1, first row) triples."""
    total = int(sum(filled))
    out, e0, row0, acc = [], 0, 0, 0
    for e, n in enumerate(filled):
        acc += int(n)
        if acc * parts >= total * (len(out) + 1) and len(out) < parts - 1:
            out.append((e0, e + 1, row0))
            e0, row0 = e + 1, acc
    out.append((e0, len(filled), row0))
    return [r for r in out if r[1] > r[0]]


def cpu_baseline(w: W.Workload, seconds: float, epilogue: str | None = None) -> dict:
    """Time the CPU oracle, unchanged, on the first min(T, 2048) tokens of
    the workload: route, slots, pack, combine (with the residual + RMSNorm
    epilogue and its fp8 encoding if `epilogue` says so), repeated for about
    `seconds` per leg.  The host-cores leg runs the oracle's own functions on
    disjoint token ranges (route, combine) and expert ranges (pack) in
    threads; slot assignment stays one serial call.  The one-thread leg runs
    each function once over the whole sample."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import oracle

    ts = min(w.T, 2048)
    ws = w.with_(T=ts, C=min(w.C, ts))
    logits = np.ascontiguousarray(W.make_logits(w)[:ts].numpy())
    x = np.ascontiguousarray(W.bits(W.make_x(w)[:ts]))
    y_pairs = np.ascontiguousarray(W.bits(W.make_y_pairs(w, rows=ts * w.k)))
    residual = x                     # any bf16 rows of the right shape
    gamma = np.ascontiguousarray(x[0])
    dtype = oracle.FP8_E4M3 if w.fp8 else oracle.BF16

    def one_thread():
        idx, wt = oracle.route_topk(logits, ws.k)
        counts, token_slot, recv_src = oracle.assign_slots(idx, ws.E, ws.C)
        oracle.pack(x, dtype, recv_src, counts, ws.C)
        if epilogue:
            _, normed = oracle.combine_residual_rmsnorm(y_pairs, token_slot, wt, residual, gamma, 1e-6)
            if epilogue == "rmsnorm-fp8":
                oracle.quantize_rows_fp8(normed)
        else:
            oracle.combine(y_pairs, token_slot, wt)

    nthr = host_threads()
    pool = ThreadPoolExecutor(nthr)
    bounds = [(ts * i // nthr, ts * (i + 1) // nthr) for i in range(nthr)]

    def threaded():
        idx = np.empty((ts, ws.k), np.int32)
        wt = np.empty((ts, ws.k), np.float32)
        list(pool.map(lambda b: oracle.route_topk_range(logits, ws.k, idx, wt, *b), bounds))
        counts, token_slot, recv_src = oracle.assign_slots(idx, ws.E, ws.C)
        filled = np.minimum(counts, ws.C)
        R = int(filled.sum())
        rows = np.empty((R, ws.H), np.uint16 if dtype == oracle.BF16 else np.uint8)
        scales = None if dtype == oracle.BF16 else np.empty((R, ws.H // 128), np.float32)
        slot_of_row = np.empty(R, np.int32)
        ranges = _balanced_expert_ranges(filled, nthr)
        list(pool.map(lambda r: oracle.pack_range(x, dtype, recv_src, counts, ws.C, rows, scales, slot_of_row,
                                                  *r), ranges))
        if epilogue:
            res_out = np.empty((ts, ws.H), np.uint16)
            normed = np.empty((ts, ws.H), np.uint16)
            list(pool.map(lambda b: oracle.combine_residual_rmsnorm_range(
                y_pairs, token_slot, wt, residual, gamma, 1e-6, res_out, normed, *b), bounds))
            if epilogue == "rmsnorm-fp8":
                q = np.empty((ts, ws.H), np.uint8)
                sc = np.empty((ts, ws.H // 128), np.float32)
                list(pool.map(lambda b: oracle.quantize_rows_fp8_range(normed, q, sc, *b), bounds))
        else:
            out = np.empty((ts, ws.H), np.uint16)
            list(pool.map(lambda b: oracle.combine_range(y_pairs, token_slot, wt, out, *b), bounds))

    def timed(fn):
        passes, t0 = 0, time.perf_counter()
        while True:
            fn()
            passes += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                return passes, el

    p1, e1 = timed(one_thread)
    pn, en = timed(threaded)
    pool.shutdown()
    nbytes = algorithmic_bytes(ws, epilogue)["total"]
    what = f"route+slots+pack+combine{EPILOGUE_LABEL[epilogue]} over the first {ts} of {w.T} tokens ({w.name})"
    return {
        "value": pn * ts / en, "unit": "tokens/s", "cores": nthr, "kind": "oracle",
        "sample": f"{pn} passes of {what} in {en:.1f} s on {nthr} threads (tokens and experts split over threads, "
                  f"slot assignment serial)",
        "gbps": nbytes * pn / en / 1e9,
        "single_thread": {"value": p1 * ts / e1, "unit": "tokens/s", "cores": 1, "gbps": nbytes * p1 / e1 / 1e9,
                          "sample": f"{p1} passes of {what} in {e1:.1f} s on one thread"},
        "host": f"{host_cpu()}, {os.cpu_count()} threads visible, {nthr} used",
    }


def floor_lib():
    """The copy-floor kernels (bench_floor.hip), built next to this file on
    first use."""
    import ctypes
    if not os.path.exists(FLOOR_LIB):
        build_floor()
    lib = ctypes.CDLL(FLOOR_LIB)
    P, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.floor_scatter_rows.argtypes = [P, i64, i32, i32, P, i32, P, P, P]
    lib.floor_scatter_rows.restype = ctypes.c_int
    lib.floor_gather_rows.argtypes = [P, i64, i32, P, P, i64, i32, P, P]
    lib.floor_gather_rows.restype = ctypes.c_int
    lib.floor_scatter_writes.argtypes = [i64, i32, i32, P, i32, P, P, P]
    lib.floor_scatter_writes.restype = ctypes.c_int
    return lib


def build_floor() -> str:
    """Compile bench_floor.hip for gfx950 into bench_floor.so."""
    hipcc = "hipcc" if subprocess.run(["which", "hipcc"], capture_output=True).returncode == 0 else "/opt/rocm/bin/hipcc"
    tmp = FLOOR_LIB + ".tmp%d" % os.getpid()
    subprocess.run([hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-fvisibility=hidden",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", FLOOR_SRC, "-o", tmp],
                   check=True, capture_output=True)
    os.replace(tmp, FLOOR_LIB)
    return FLOOR_LIB


class BufferSet:
    """One complete copy of a step's inputs, outputs and fixed-slot buffers."""

    def __init__(self, w: W.Workload, logits_cpu, x_cpu, dev, moe, torch, route_groups=None, packed=False,
                 epilogue=None, fuse_route=True):
        self.fuse_route = fuse_route
        self.packed = packed
        self.logits = logits_cpu.to(dev)
        self.x = x_cpu.to(dev)
        self.idx = torch.empty(w.T, w.k, dtype=torch.int32, device=dev)
        self.wt = torch.empty(w.T, w.k, dtype=torch.float32, device=dev)
        if packed:
            self.bufs = moe.PackedBuffers.allocate(w.T, w.H, w.E, w.k, w.fp8, dev)
            self.y = torch.empty(w.T * w.k, w.H, dtype=torch.bfloat16, device=dev)
        else:
            self.bufs = moe.DispatchBuffers.allocate(w.T, w.H, w.E, w.k, w.C, w.fp8, dev)
            self.y = torch.empty(w.E, w.C, w.H, dtype=torch.bfloat16, device=dev)
        self.out = torch.empty(w.T, w.H, dtype=torch.bfloat16, device=dev)
        self.epilogue = None
        if epilogue:
            # residual stream (a copy of the activations, in its own memory: were
            # it x itself, the next step's pack would find x in the last-level
            # cache, freshly read by this combine) and RMSNorm weight
            residual = self.x.clone()
            gamma = torch.linspace(0.5, 1.5, w.H, device=dev).to(torch.bfloat16)
            self.epilogue = (residual, gamma, 1e-6, torch.empty(w.T, w.H, dtype=torch.bfloat16, device=dev))
            if epilogue == "rmsnorm-fp8":
                self.epilogue += (torch.empty(w.T, w.H, dtype=torch.uint8, device=dev),
                                  torch.empty(w.T, w.H // 128, dtype=torch.float32, device=dev))
        self.route_groups = route_groups
        self.step = self.prepare(w, moe)

    def prepare(self, w, moe, stream=None):
        return moe.PreparedStep(self.logits, w.k, self.x, w.C, w.fp8, self.bufs, self.y, self.out, self.idx,
                                self.wt, stream=stream, route_groups=self.route_groups, epilogue=self.epilogue,
                                fuse_route=self.fuse_route)

    def fill_expert_outputs(self, w: W.Workload, torch, gen):
        """Seeded N(0,1) bf16 expert outputs in the slots the dispatch filled."""
        slots = self.bufs.token_slot.reshape(-1)
        slots = slots[slots >= 0].to(torch.int64)
        rows = torch.randn(slots.numel(), w.H, device=self.y.device, generator=gen, dtype=torch.float32)
        self.y.view(-1, w.H).index_copy_(0, slots, rows.to(torch.bfloat16))


def _stats_us(v_ms):
    v = sorted(x * 1e3 for x in v_ms)
    return {"mean_us": sum(v) / len(v), "median_us": v[len(v) // 2], "min_us": v[0], "max_us": v[-1],
            "launches": len(v)}


def run_workload(w: W.Workload, args, moe, torch, dev, primary: bool) -> dict:
    """Headline timing, kernel timing pass, copy floors (and for the primary
    workload the graph-replay and two-stream extras) of one workload."""
    epilogue = None if args.epilogue == "none" else args.epilogue
    nbytes = algorithmic_bytes(w, epilogue)
    K = args.steps if args.steps > 0 else (200 if w.T <= 4096 else 50)
    Wm = args.warmup
    R = args.rotate or max(1, min(32, math.ceil(2 * 2 ** 30 / nbytes["total"])))
    S = max(1, args.streams) if primary else 1
    if R % S:
        R += S - R % S

    logits_cpu = W.make_logits(w)
    x_cpu = W.make_x(w)
    route_groups = tuple(int(v) for v in args.route_groups.split(":")) if args.route_groups else None
    packed = args.layout == "packed"
    fuse_route = not args.separate_route and route_groups is None
    sets = [BufferSet(w, logits_cpu, x_cpu, dev, moe, torch, route_groups, packed, epilogue, fuse_route)
            for _ in range(R)]
    del logits_cpu, x_cpu
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed * 16 + 3)
    for s in sets:
        s.step.route_and_dispatch()
        s.fill_expert_outputs(w, torch, gen)
    torch.cuda.synchronize()

    main = torch.cuda.current_stream()
    streams = [main] + [torch.cuda.Stream() for _ in range(max(S, 2) - 1)]
    hip_events = moe.HipEvents()

    def bind(nstreams):
        """Bind buffer set i to stream i % nstreams (a set never changes stream
        while steps are queued)."""
        torch.cuda.synchronize()
        for si, st in enumerate(sets):
            st.step = st.prepare(w, moe, stream=streams[si % nstreams])

    def run_steps(first, n, nstreams):
        for i in range(n):
            st = sets[(first + i) % R].step
            st.route_and_dispatch()
            st.combine()

    def timed(first, n, nstreams):
        torch.cuda.synchronize()
        for strm in streams[1:nstreams]:
            strm.wait_stream(main)
        t0 = time.perf_counter()
        run_steps(first, n, nstreams)
        for strm in streams[1:nstreams]:
            main.wait_stream(strm)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / n

    # headline: K steps with nothing but the steps in the stream(s)
    bind(S)
    run_steps(0, Wm, S)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(main)
    ms = timed(Wm, K, S)
    e1.record(main)
    torch.cuda.synchronize()
    event_ms = e0.elapsed_time(e1) / K     # includes the trailing sync gap; reported only
    gbps = nbytes["total"] / (ms * 1e-3) / 1e9

    # kernel timing pass (after the headline region, one stream): HIP events
    # recorded on the launch stream around every call.  Where moe_route_dispatch
    # launches the same kernels as moe_route_topk + moe_dispatch, the two calls
    # are made and timed separately: grouped routing, and E > 8 at the
    # benchmark's sizes (decode is counted inside pack, and the prefill
    # batches are past the size up to which the fused call's router writes
    # membership words instead).
    bind(1)
    split = w.E > 8 or route_groups is not None or args.separate_route
    n = min(K, 200)
    marks = [tuple(hip_events.create() for _ in range(4)) for _ in range(n)]
    torch.cuda.synchronize()
    for i, (a, b, c, d) in enumerate(marks):
        st = sets[(Wm + K + i) % R].step
        hip_events.record(a, main)
        if split:
            st.route()
            hip_events.record(b, main)
            st.dispatch()
        else:
            st.route_and_dispatch()
        hip_events.record(c, main)
        st.combine()
        hip_events.record(d, main)
    torch.cuda.synchronize()
    comb = [hip_events.elapsed_ms(c, d) for _, _, c, d in marks]
    kernels = {}
    if split:
        route = [hip_events.elapsed_ms(a, b) for a, b, _, _ in marks]
        disp = [hip_events.elapsed_ms(b, c) for _, b, c, _ in marks]
        kernels["route"] = {"call": "moe_route_topk" + ("_grouped" if route_groups else ""),
                            "bytes": nbytes["route"], **_stats_us(route)}
        kernels["dispatch"] = {"call": "moe_dispatch" + ("_packed" if packed else "") + " (count + pack launches)",
                               "bytes": nbytes["count_scan_slot"] + nbytes["pack"], **_stats_us(disp)}
    else:
        rd = [hip_events.elapsed_ms(a, c) for a, _, c, _ in marks]
        kernels["route_dispatch"] = {"call": "moe_route_dispatch" + ("_packed" if packed else ""),
                                     "bytes": nbytes["route"] + nbytes["count_scan_slot"] + nbytes["pack"],
                                     **_stats_us(rd)}
    kernels["combine"] = {"call": {None: "moe_combine", "rmsnorm": "moe_combine_residual_rmsnorm",
                                   "rmsnorm-fp8": "moe_combine_residual_rmsnorm_fp8"}[epilogue],
                          "bytes": nbytes["combine"], **_stats_us(comb)}
    for kv in kernels.values():
        kv["gbps"] = kv["bytes"] / (kv["mean_us"] * 1e-6) / 1e9
        kv["frac"] = kv["gbps"] / HBM_PEAK_GBPS
    for trio in marks:
        for e in trio:
            hip_events.destroy(e)

    # copy floors: plain kernels moving pack's and combine's exact bytes, and
    # pack's stores alone
    floor = None
    if not args.no_floor and not epilogue:
        lib = floor_lib()
        fl_events = [tuple(hip_events.create() for _ in range(6)) for _ in range(n)]
        s0 = main.cuda_stream

        def floor_run(st, ev=None):
            bf = st.bufs
            scales = bf.recv_scales.data_ptr() if w.fp8 else None
            if ev:
                hip_events.record(ev[0], main)
            rc = lib.floor_scatter_rows(st.x.data_ptr(), w.T, w.H, int(w.fp8), bf.token_slot.data_ptr(), w.k,
                                        bf.recv_x.data_ptr(), scales, s0)
            if ev:
                hip_events.record(ev[1], main)
                hip_events.record(ev[2], main)
            rc |= lib.floor_gather_rows(st.y.data_ptr(), st.y.numel() // w.H, w.H, bf.token_slot.data_ptr(),
                                        st.wt.data_ptr(), w.T, w.k, st.out.data_ptr(), s0)
            if ev:
                hip_events.record(ev[3], main)
                hip_events.record(ev[4], main)
            rc |= lib.floor_scatter_writes(w.T, w.H, int(w.fp8), bf.token_slot.data_ptr(), w.k,
                                           bf.recv_x.data_ptr(), scales, s0)
            if ev:
                hip_events.record(ev[5], main)
            if rc:
                raise RuntimeError(f"copy-floor launch failed ({rc})")

        floor_run(sets[0])           # untimed: the first launch also loads the kernels' code
        torch.cuda.synchronize()
        for i, ev in enumerate(fl_events):
            floor_run(sets[(Wm + K + n + i) % R], ev)
        torch.cuda.synchronize()
        sc = _stats_us([hip_events.elapsed_ms(e[0], e[1]) for e in fl_events])
        ga = _stats_us([hip_events.elapsed_ms(e[2], e[3]) for e in fl_events])
        wo = _stats_us([hip_events.elapsed_ms(e[4], e[5]) for e in fl_events])
        for e6 in fl_events:
            for e in e6:
                hip_events.destroy(e)
        # a plain sequential fill of one receive buffer: its bandwidth for
        # writes that are not scattered
        rx = sets[0].bufs.recv_x
        fill_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        rx.fill_(0)
        torch.cuda.synchronize()
        fill_ev[0].record(main)
        for _ in range(3):
            rx.fill_(0)
        fill_ev[1].record(main)
        torch.cuda.synchronize()
        fill_us = fill_ev[0].elapsed_time(fill_ev[1]) * 1e3 / 3
        fill_bytes = rx.numel() * rx.element_size()
        pack_bytes = nbytes["pack"]
        write_bytes = w.T * w.k * ((w.H + w.H // 32) if w.fp8 else 2 * w.H)
        floor = {
            "pack_shaped_copy": {"kernel": "floor_scatter_rows (bench_floor.hip)", "bytes": pack_bytes, **sc,
                                 "gbps": pack_bytes / (sc["mean_us"] * 1e-6) / 1e9},
            "combine_shaped_copy": {"kernel": "floor_gather_rows (bench_floor.hip)", "bytes": nbytes["combine"],
                                    **ga, "gbps": nbytes["combine"] / (ga["mean_us"] * 1e-6) / 1e9},
            "pack_writes_only": {"kernel": "floor_scatter_writes (bench_floor.hip)", "bytes": write_bytes, **wo,
                                 "gbps": write_bytes / (wo["mean_us"] * 1e-6) / 1e9},
            "receive_buffer_fill": {"kernel": "torch fill_ of one receive buffer (sequential writes)",
                                    "bytes": fill_bytes, "mean_us": fill_us,
                                    "gbps": fill_bytes / (fill_us * 1e-6) / 1e9},
            "note": "plain copies of the same rows at the same addresses (no slot work, no quantisation, no "
                    "arithmetic); their bytes are pack's and combine's algorithmic bytes. pack_writes_only: the "
                    "copy's stores without its reads; receive_buffer_fill: the same memory written sequentially",
        }
        for v in floor.values():
            if isinstance(v, dict):
                v["frac"] = v["gbps"] / HBM_PEAK_GBPS

    res = {
        "workload": w.name, "tokens": w.T, "hidden": w.H, "experts": w.E, "top_k": w.k, "capacity": w.C,
        "row_dtype": "fp8-e4m3+fp32/128" if w.fp8 else "bf16", "routing": w.routing,
        "steps": K, "warmup": Wm, "ms_per_step": ms, "tokens_per_s": w.T / (ms * 1e-3),
        "algorithmic_bytes_per_step": nbytes["total"], "effective_hbm_gbps": gbps, "hbm_frac": gbps / HBM_PEAK_GBPS,
        "buffer_copies_cycled": R, "streams": S, "ms_per_step_events": event_ms,
        "kernels": kernels, "floor": floor,
    }

    if primary:
        # the same steps replayed from HIP graphs (one captured step per buffer
        # set): no host launch cost, so small batches show their GPU time
        if not args.no_graph and S == 1:
            cap = torch.cuda.Stream()
            torch.cuda.synchronize()
            for st in sets:
                st.step = st.prepare(w, moe, stream=cap)
            graphs = []
            for st in sets:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=cap):
                    st.step.route_and_dispatch()
                    st.step.combine()
                graphs.append(g)
            for i in range(Wm):
                graphs[i % R].replay()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(K):
                graphs[(Wm + i) % R].replay()
            torch.cuda.synchronize()
            g_ms = (time.perf_counter() - t0) * 1e3 / K
            res["graph_replay"] = {"ms_per_step": g_ms, "tokens_per_s": w.T / (g_ms * 1e-3),
                                   "hbm_frac": nbytes["total"] / (g_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS}
            del graphs
        # two independent batches in flight (steps alternate over two streams)
        if not args.no_overlap and S == 1 and R >= 2:
            bind(2)
            run_steps(0, Wm, 2)
            ov_ms = timed(Wm, K, 2)
            res["two_batches_in_flight"] = {"streams": 2, "ms_per_step": ov_ms, "tokens_per_s": w.T / (ov_ms * 1e-3),
                                            "hbm_frac": nbytes["total"] / (ov_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS}
        res.update({
            "route_groups": ({"groups": route_groups[0], "kept": route_groups[1]} if route_groups else None),
            "layout": "packed count-sized rows" if packed else "fixed slots per expert",
            "route_dispatch_call": (("moe_route_dispatch_packed" if packed else "moe_route_dispatch") if fuse_route
                                    else "separate"),
            "combine_epilogue": {None: None, "rmsnorm": "residual add + RMSNorm (fused)",
                                 "rmsnorm-fp8": "residual add + RMSNorm, output as E4M3 + fp32/128 (fused)"}[epilogue],
        })
        res["_traffic"] = None if (packed or epilogue) else measured_traffic(w)

    del sets
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def placement_probe(w: W.Workload, n_recv: int, moe, torch, dev) -> dict:
    """The same dispatch and combine calls on separately allocated buffers, in
    one process: `n_recv` receive buffers (codes or rows, scales and the small
    outputs, each its own allocation) and max(1, n_recv // 2) expert-output
    buffers, each timed over two passes of 10 calls, beside a plain
    sequential fill of the same buffer; then dispatch into the first receive
    buffer viewed with other per-expert capacities (strides).  Inputs, ids and
    weights are shared, so the buffers' memory is the only difference."""
    logits = W.make_logits(w).to(dev)
    x = W.make_x(w).to(dev)
    idx, wt = moe.moe_route_topk(logits, w.k)
    max_count = int(torch.bincount(idx.view(-1).long(), minlength=w.E).max())
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def per_call_us(fn, n=10):
        fn()
        torch.cuda.synchronize()
        ev0.record()
        for _ in range(n):
            fn()
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) * 1e3 / n

    def fill_tbps(t):
        us = per_call_us(lambda: t.fill_(1), n=3)
        return t.numel() * t.element_size() / (us * 1e-6) / 1e12

    caps = sorted({w.C, w.C + 1, w.C + 16, w.C + 1024, -(-max_count // 256) * 256})
    cmax = max(caps)
    recv = []
    for i in range(n_recv):
        b = moe.DispatchBuffers.allocate(w.T, w.H, w.E, w.k, cmax if i == 0 else w.C, w.fp8, dev)
        recv.append(b)

    def dispatch_into(b, C):
        rows = w.E * C
        view = moe.DispatchBuffers(
            recv_x=b.recv_x.view(-1)[:rows * w.H].view(w.E, C, w.H),
            recv_scales=(b.recv_scales.view(-1)[:rows * (w.H // 128)].view(w.E, C, w.H // 128) if w.fp8 else None),
            recv_src=b.recv_src.view(-1)[:rows].view(w.E, C), expert_counts=b.expert_counts,
            token_slot=b.token_slot, workspace=b.workspace)
        return lambda: moe.moe_route_dispatch(logits, x, w.k, C, fp8=w.fp8, bufs=view, topk_idx=idx, topk_w=wt)

    res = {"workload": w.name, "call": "moe_route_dispatch", "max_expert_count": max_count, "receive_buffers": []}
    for i, b in enumerate(recv):
        C = w.C
        res["receive_buffers"].append({
            "capacity": C, "dispatch_us": [round(per_call_us(dispatch_into(b, C)), 1) for _ in range(2)],
            "sequential_fill_tbps": round(fill_tbps(b.recv_x), 2)})
    res["capacity_sweep_first_buffer_us"] = {str(C): round(per_call_us(dispatch_into(recv[0], C)), 1) for C in caps}
    slots = recv[-1].token_slot
    out = torch.empty(w.T, w.H, dtype=torch.bfloat16, device=dev)
    res["expert_output_buffers"] = []
    ys = []   # all kept alive, so that each is a fresh allocation
    for _ in range(max(1, n_recv // 2)):
        y = torch.empty(w.E, w.C, w.H, dtype=torch.bfloat16, device=dev)
        ys.append(y)
        res["expert_output_buffers"].append({
            "combine_us": [round(per_call_us(lambda: moe.moe_combine(y, slots, wt, out=out)), 1) for _ in range(2)],
            "sequential_fill_tbps": round(fill_tbps(y), 2)})
    return res


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=0,
                    help="timed steps (default 200 for batches of at most 4096 tokens, else 50)")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=W.ORDER)
    ap.add_argument("--also", default="auto",
                    help="comma-separated workloads measured after the headline one and reported in "
                         "config.other_workloads; 'auto' = the other prefill workloads when the headline is the "
                         "default one; 'none' = no others")
    ap.add_argument("--rotate", type=int, default=0,
                    help="buffer copies cycled through (0: enough that 2 GiB of step traffic separates reuses)")
    ap.add_argument("--cpu-seconds", type=float, default=8.0, help="seconds per CPU baseline leg")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--streams", type=int, default=1,
                    help="HIP streams the timed steps alternate over (2: two independent batches in flight)")
    ap.add_argument("--no-overlap", action="store_true",
                    help="skip the extra two-batches-in-flight measurement")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the extra HIP-graph-replay measurement")
    ap.add_argument("--no-floor", action="store_true",
                    help="skip the copy floors (plain copies of pack's and combine's bytes)")
    ap.add_argument("--layout", choices=["fixed", "packed"], default="fixed",
                    help="dispatch layout: fixed slots per expert (moe_dispatch) or packed count-sized rows "
                         "(moe_dispatch_packed)")
    ap.add_argument("--epilogue", choices=["none", "rmsnorm", "rmsnorm-fp8"], default="none",
                    help="combine with the fused residual add + RMSNorm (moe_combine_residual_rmsnorm), or "
                         "with its rows written as E4M3 + per-128 scales (moe_combine_residual_rmsnorm_fp8)")
    ap.add_argument("--separate-route", action="store_true",
                    help="call moe_route_topk and moe_dispatch separately instead of moe_route_dispatch")
    ap.add_argument("--route-groups", default="",
                    help="G:M routes with moe_route_topk_grouped (G expert groups, the best M kept)")
    ap.add_argument("--placement", type=int, default=0,
                    help="instead of the benchmark: time moe_route_dispatch and moe_combine (fixed-slot layout) "
                         "on this many separately allocated receive buffers (and half as many expert-output "
                         "buffers) of the workload, plus a capacity sweep; prints one JSON object")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this path has no multi-GPU (sharded) mode; run with --gpus 1",
              file=sys.stderr)
        return 2

    import torch

    import combine_moe_route_amd as moe

    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        return 1
    moe.load()
    dev = torch.device("cuda:0")
    w = W.WORKLOADS[args.workload]
    if args.placement:
        print(json.dumps({"placement": placement_probe(w, args.placement, moe, torch, dev)}), flush=True)
        return 0
    epilogue = None if args.epilogue == "none" else args.epilogue
    if args.also == "auto":
        others = [n for n in SECONDARY if n != w.name] if w.name == DEFAULT_WORKLOAD else []
    elif args.also == "none":
        others = []
    else:
        others = [n for n in args.also.split(",") if n]

    def summary(r):
        line = f"# {r['workload']}: {r['ms_per_step'] * 1e3:.1f} us/step, {r['hbm_frac']:.3f} of 8 TB/s"
        fl = r.get("floor") or {}
        if "pack_writes_only" in fl:
            line += (f"; pack's stores alone {fl['pack_writes_only']['gbps'] / 1e3:.2f} TB/s, receive buffer "
                     f"sequential fill {fl['receive_buffer_fill']['gbps'] / 1e3:.2f} TB/s")
        print(line, file=sys.stderr, flush=True)

    head = run_workload(w, args, moe, torch, dev, primary=True)
    summary(head)
    other = []
    for name in others:
        r = run_workload(W.WORKLOADS[name], args, moe, torch, dev, primary=False)
        summary(r)
        other.append(r)

    if args.copy_mib:
        n = args.copy_mib * 2 ** 20
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty(n, dtype=torch.uint8, device=dev)
        a.fill_(1)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    ms = head["ms_per_step"]
    comb = head["kernels"]["combine"]
    traffic = head.pop("_traffic", None)
    config = {k: v for k, v in head.items() if k not in ("steps", "warmup", "ms_per_step")}
    config["parallelism"] = "none (1 GPU)"
    config["other_workloads"] = other
    result = {
        "metric": METRIC,
        "value": w.T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": head["steps"],
        "warmup": head["warmup"],
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": config,
        "roofline": {
            "kernel": (f"{comb['call']} (k={w.k}); profiles/{w.name}_kernel_trace.md names the kernel instance"),
            "bound": "hbm",
            "achieved": comb["gbps"],
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": comb["frac"],
            "traffic": traffic,
            "traffic_source": f"profiles/{w.name}_hbm_traffic.md (bytes per launch)",
            "algorithmic_bytes_per_launch": comb["bytes"],
            "mean_launch_us": comb["mean_us"],
            "median_launch_us": comb["median_us"],
            "min_launch_us": comb["min_us"],
            "max_launch_us": comb["max_us"],
            "timed_launches": comb["launches"],
            "timing": "HIP events recorded on the launch stream around every combine call of a timing pass run "
                      "after the (event-free) headline region",
        },
    }
    # the other HBM-bound call of the step, timed the same way
    dname = "dispatch" if "dispatch" in head["kernels"] else "route_dispatch"
    disp = head["kernels"][dname]
    result["roofline_dispatch"] = {
        "kernel": f"{disp['call']}; profiles/{w.name}_kernel_trace.md names the kernel instances",
        "bound": "hbm", "achieved": disp["gbps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": disp["frac"],
        "algorithmic_bytes_per_launch": disp["bytes"], "mean_launch_us": disp["mean_us"],
        "median_launch_us": disp["median_us"], "timed_launches": disp["launches"],
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, epilogue)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

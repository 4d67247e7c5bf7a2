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
W untimed warm-up steps, then exactly K timed steps between device
synchronisations.  Prints one JSON line (stdout):

  value     tokens/s of the whole job (one GPU)
  config    the workload plus effective HBM GB/s and fraction of the 8 TB/s
            peak, from the algorithmic byte model (each row read once and
            written k times, unfilled slots not counted)
  roofline  the dominant kernel (combine): algorithmic bytes per launch over
            its mean launch time from HIP events recorded around each launch
            in the timed region, against the 8 TB/s HBM peak
  cpu_baseline  the CPU oracle (single-threaded, plain C) on a bounded
            sample of the same workload

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
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

METRIC = "dispatch+combine tokens/s and effective HBM GB/s (% of peak), 1 MI355X"
EPILOGUE_LABEL = {None: "", "rmsnorm": "+residual+rmsnorm", "rmsnorm-fp8": "+residual+rmsnorm+fp8"}
HBM_PEAK_GBPS = 8000.0
LLC_BYTES = 256 * 2 ** 20


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


def cpu_baseline(w: W.Workload, seconds: float, epilogue: str | None = None) -> dict:
    """Time the CPU oracle (route, slots, pack, combine -- with the residual
    + RMSNorm epilogue, and its fp8 encoding, if `epilogue` says so) on the
    first min(T, 2048) tokens of the workload, repeated for ~`seconds`."""
    import numpy as np
    import oracle

    ts = min(w.T, 2048)
    ws = w.with_(T=ts, C=min(w.C, ts))
    logits = W.make_logits(w)[:ts].numpy()
    x = W.bits(W.make_x(w)[:ts])
    y_pairs = W.bits(W.make_y_pairs(w, rows=ts * w.k))
    residual = x                     # any bf16 rows of the right shape
    gamma = x[0]
    passes, t0 = 0, time.perf_counter()
    while True:
        idx, wt = oracle.route_topk(logits, ws.k)
        counts, token_slot, recv_src = oracle.assign_slots(idx, ws.E, ws.C)
        oracle.pack(x, oracle.FP8_E4M3 if w.fp8 else oracle.BF16, recv_src, counts, ws.C)
        if epilogue:
            _, normed = oracle.combine_residual_rmsnorm(y_pairs, token_slot, wt, residual, gamma, 1e-6)
            if epilogue == "rmsnorm-fp8":
                oracle.quantize_rows_fp8(normed)
        else:
            oracle.combine(y_pairs, token_slot, wt)
        passes += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    tok_s = passes * ts / el
    return {
        "value": tok_s, "unit": "tokens/s", "cores": 1, "kind": "oracle",
        "sample": f"{passes} passes of route+slots+pack+combine{EPILOGUE_LABEL[epilogue]} over the "
                  f"first {ts} of {w.T} tokens ({w.name}), {el:.1f} s",
        "gbps": algorithmic_bytes(ws, epilogue)["total"] * passes / el / 1e9,
        "host": f"{host_cpu()}, {os.cpu_count()} threads visible",
    }


class BufferSet:
    """One complete copy of a step's inputs, outputs and fixed-slot buffers."""

    def __init__(self, w: W.Workload, logits_cpu, x_cpu, dev, moe, torch, route_groups=None, packed=False,
                 epilogue=None, fuse_route=True):
        self.fuse_route = fuse_route
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
            # residual stream (the activations stand in for it) and RMSNorm weight
            gamma = torch.linspace(0.5, 1.5, w.H, device=dev).to(torch.bfloat16)
            self.epilogue = (self.x, gamma, 1e-6, torch.empty(w.T, w.H, dtype=torch.bfloat16, device=dev))
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


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=0,
                    help="timed steps (default 200 for batches of at most 4096 tokens, else 50)")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mixtral_prefill", choices=W.ORDER)
    ap.add_argument("--rotate", type=int, default=0,
                    help="buffer copies cycled through (0: enough that 2 GiB of step traffic separates reuses)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--streams", type=int, default=1,
                    help="HIP streams the timed steps alternate over (2: two independent batches in flight)")
    ap.add_argument("--timing", choices=["ext", "marker"], default="ext",
                    help="combine launch timing: events attached to the launch (ext) or recorded around it")
    ap.add_argument("--no-overlap", action="store_true",
                    help="skip the extra two-batches-in-flight measurement")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the extra HIP-graph-replay measurement")
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
    if args.steps <= 0:
        args.steps = 200 if w.T <= 4096 else 50
    epilogue = None if args.epilogue == "none" else args.epilogue
    if epilogue:
        args.timing = "marker"       # the fused kernel has no launch-attached timing entry point
    nbytes = algorithmic_bytes(w, epilogue)
    R = args.rotate or max(1, min(32, math.ceil(2 * 2 ** 30 / nbytes["total"])))

    logits_cpu = W.make_logits(w)
    x_cpu = W.make_x(w)
    route_groups = tuple(int(v) for v in args.route_groups.split(":")) if args.route_groups else None
    packed = args.layout == "packed"
    fuse_route = not args.separate_route and route_groups is None
    sets = [BufferSet(w, logits_cpu, x_cpu, dev, moe, torch, route_groups, packed, epilogue, fuse_route)
            for _ in range(R)]
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed * 16 + 3)
    for s in sets:
        s.step.route_and_dispatch()
        s.fill_expert_outputs(w, torch, gen)
    torch.cuda.synchronize()

    K, Wm = args.steps, args.warmup
    S = max(1, args.streams)
    main = torch.cuda.current_stream()
    streams = [main] + [torch.cuda.Stream() for _ in range(max(S, 2) - 1)]
    hip_events = moe.HipEvents()

    def bind(nstreams):
        """Bind buffer set i to stream i % nstreams (a set never changes stream
        while steps are queued)."""
        torch.cuda.synchronize()
        for si, st in enumerate(sets):
            st.step = st.prepare(w, moe, stream=streams[si % nstreams])

    def run_steps(first, n, nstreams, ev=None):
        """n steps over buffer sets first, first+1, ...; when `ev` maps step
        index -> (start, stop) raw events, those steps' combine launches are
        timed."""
        for i in range(n):
            si = (first + i) % R
            st = sets[si].step
            st.route_and_dispatch()
            pair = ev.get(i) if ev else None
            if pair is None:
                st.combine()
            elif args.timing == "ext":
                st.combine_timed(*pair)
            else:
                hip_events.record(pair[0], streams[si % nstreams])
                st.combine()
                hip_events.record(pair[1], streams[si % nstreams])

    def timed(first, n, nstreams, ev=None):
        torch.cuda.synchronize()
        for strm in streams[1:nstreams]:
            strm.wait_stream(main)
        t0 = time.perf_counter()
        run_steps(first, n, nstreams, ev)
        for strm in streams[1:nstreams]:
            main.wait_stream(strm)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / n

    # headline: S stream(s), combine timed per launch by its own kernel timestamps
    if R % S:
        R -= R % S
    bind(S)
    run_steps(0, Wm, S)
    # every event pair is a pair of barrier packets in the stream (~3.5 us of
    # lost pipelining each on this runtime), so only ~8 launches spread over
    # the K timed steps carry them
    every = max(1, K // 8)
    ev = {i: (hip_events.create(), hip_events.create()) for i in range(every // 2, K, every)}
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(main)
    wall_ms = timed(Wm, K, S, ev)
    e1.record(main)
    torch.cuda.synchronize()
    event_ms = e0.elapsed_time(e1) / K     # includes the trailing sync gap; reported only
    ms = wall_ms
    combine_times = [hip_events.elapsed_ms(a, b) for a, b in ev.values()]
    combine_ms = sum(combine_times) / len(combine_times)
    for a, b in ev.values():
        hip_events.destroy(a)
        hip_events.destroy(b)

    # the same steps without timing events, for comparison
    plain_ms = timed(Wm + K, K, S)

    # each call alone: events recorded around route + dispatch and around
    # combine for ~K/4 steps, a pass of its own outside the timed region
    per_call = None
    if S == 1:
        n = max(8, K // 4)
        marks = [(hip_events.create(), hip_events.create(), hip_events.create()) for _ in range(n)]
        torch.cuda.synchronize()
        for i, (a, b, c) in enumerate(marks):
            st = sets[(Wm + 2 * K + i) % R].step
            hip_events.record(a, main)
            st.route_and_dispatch()
            hip_events.record(b, main)
            st.combine()
            hip_events.record(c, main)
        torch.cuda.synchronize()

        def stats(v):
            v = sorted(x * 1e3 for x in v)
            return {"median": v[len(v) // 2], "min": v[0], "max": v[-1]}
        per_call = {"steps": n,
                    "route_dispatch_us": stats([hip_events.elapsed_ms(a, b) for a, b, _ in marks]),
                    "combine_us": stats([hip_events.elapsed_ms(b, c) for _, b, c in marks]),
                    "timing": "device-release HIP events recorded around each call, one step at a time"}
        for trio in marks:
            for e in trio:
                hip_events.destroy(e)

    # the same steps replayed from HIP graphs (one captured step per buffer
    # set): no host launch cost, so small batches show their GPU time
    graph = None
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
        graph = {"ms_per_step": g_ms, "tokens_per_s": w.T / (g_ms * 1e-3),
                 "hbm_frac": nbytes["total"] / (g_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS}
        del graphs
        bind(S)

    # two independent batches in flight (steps alternate over two streams)
    overlap = None
    if not args.no_overlap and S == 1 and R >= 2:
        bind(2)
        run_steps(0, Wm, 2)
        ov_ms = timed(Wm, K, 2)
        overlap = {"streams": 2, "ms_per_step": ov_ms, "tokens_per_s": w.T / (ov_ms * 1e-3),
                   "hbm_frac": nbytes["total"] / (ov_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS}
    gbps = nbytes["total"] / (ms * 1e-3) / 1e9
    comb_gbps = nbytes["combine"] / (combine_ms * 1e-3) / 1e9

    if args.copy_mib:
        n = args.copy_mib * 2 ** 20
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty(n, dtype=torch.uint8, device=dev)
        a.fill_(1)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()

    result = {
        "metric": METRIC,
        "value": w.T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name, "tokens": w.T, "hidden": w.H, "experts": w.E, "top_k": w.k, "capacity": w.C,
            "row_dtype": "fp8-e4m3+fp32/128" if w.fp8 else "bf16", "routing": w.routing,
            "route_groups": ({"groups": route_groups[0], "kept": route_groups[1]} if route_groups else None),
            "layout": "packed count-sized rows" if packed else "fixed slots per expert",
            "route_dispatch_call": (("moe_route_dispatch_packed" if packed else "moe_route_dispatch") if fuse_route
                                    else "separate"),
            "combine_epilogue": {None: None, "rmsnorm": "residual add + RMSNorm (fused)",
                                 "rmsnorm-fp8": "residual add + RMSNorm, output as E4M3 + fp32/128 (fused)"}[epilogue],
            "parallelism": "none (1 GPU)",
            "algorithmic_bytes_per_step": nbytes["total"],
            "effective_hbm_gbps": gbps,
            "hbm_frac": gbps / HBM_PEAK_GBPS,
            "buffer_copies_cycled": R,
            "streams": S,
            "ms_per_step_events": event_ms,
            "ms_per_step_without_timing_events": plain_ms,
            "two_batches_in_flight": overlap,
            "graph_replay": graph,
            "per_call": per_call,
        },
        "roofline": {
            "kernel": (f"combine_rmsnorm_kernel (k={w.k}{', fp8 out' if epilogue == 'rmsnorm-fp8' else ''})"
                       if epilogue else f"moe_combine (k={w.k}); profiles/{w.name}_kernel_trace.md names the kernel"),
            "bound": "hbm",
            "achieved": comb_gbps,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": comb_gbps / HBM_PEAK_GBPS,
            "traffic": None if (packed or epilogue) else measured_traffic(w),
            "traffic_source": f"profiles/{w.name}_hbm_traffic.md (bytes per launch)",
            "algorithmic_bytes_per_launch": nbytes["combine"],
            "mean_launch_us": combine_ms * 1e3,
            "median_launch_us": sorted(combine_times)[len(combine_times) // 2] * 1e3,
            "timed_launches": len(combine_times),
            "min_launch_us": min(combine_times) * 1e3,
            "max_launch_us": max(combine_times) * 1e3,
            "timing": ("device-release HIP events attached to each timed combine launch (moe_combine_timed)"
                       if args.timing == "ext" else "device-release HIP events recorded around each timed combine"),
        },
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, epilogue)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

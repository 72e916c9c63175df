#!/usr/bin/env python3
"""Benchmark: MoE layout -> dispatch -> combine on one MI355X.

One step is one pass of the whole path over one batch of the DeepSeek-V3-style
prefill workload: T=8192 tokens, hidden 7168, 256 experts in 8 groups, top-8,
FP8 E4M3 dispatch with one fp32 scale per 128 channels, bf16 combine.  Inputs
are seeded synthetic data, resident in HBM before timing starts.  The expert
stage is an identity stand-in computed once before timing (dispatch is
deterministic, so its output is the same every step); it is not part of the
path and not timed.

Prints one JSON line.  `value` is the step's ideal (algorithmic) HBM bytes
divided by the step's wall time over K back-to-back steps with nothing else
enqueued (the steady state, in which x is still in the last-level cache from
the previous step, as it would be after the router read it).  The per-kernel
times come from a separate pass of K steps with HIP events recorded around
every call on the stream the kernels run on; the events cost a few us each,
so that pass's step time is reported apart (`ms_per_step_with_events`).

`after_flush` holds the HBM-only figures: every one of those steps starts
after a 512 MiB read has emptied L2 and the MALL.  It gives per-kernel times
(events around every call), the whole step's time with events only at its two
ends, the dispatch kernel's roofline fraction, and the same whole step with
ep_layout_dispatch and EP_READ_X_AHEAD (x read into the MALL while the
latency-bound layout runs), for the workloads where that applies.

`roofline` is the dominant kernel's (combine): algorithmic bytes per launch
over the mean HIP-event time of its launches, beside the committed rocprofv3
kernel-trace mean and HBM traffic when they were taken on the current kernel
sources; `kernel_us_profile` then gives that trace's time of every kernel of
the step (no event cost) and dispatch + combine over those times.
`cpu_baseline` is the oracle on this host's cores, single-threaded and with
the tokens split across the cores.

`--workload` times the other named workloads (tiny, skewed, lowlat, large) the
same way; the default is the configuration the metric is quoted on.  Variant
flags: --fused (one-call layout+dispatch), --read-x-ahead (the same with
EP_READ_X_AHEAD), --pow2 / --mx (power-of-two or MXFP8 scales), --mn-scales
(dispatch stores its scales transposed), --mn-convert (row-major dispatch, then
the scale-layout conversion kernel), --fp8-combine (FP8 expert outputs), --f16
(fp16 rows), --dedup (per-group dedup layout, dispatch and combine), --graph
(HIP graph).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, AMD's published figure
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "combine_moe_layout_amd", "csrc")


def ideal_bytes(T: int, H: int, E: int, G: int, k: int, R_used: int, fp8: bool,
                fp8_combine: bool = False) -> dict:
    """Algorithmic HBM bytes of one pass (each byte the path must move, once).

    layout:   read topk_idx (8 B per pair), write slot_idx (4 B per pair),
              write counts / offsets / group totals (4 B each).
    dispatch: read x once (2H B per token); per used receive row write H B of
              codes and 4*H/128 B of scales (FP8) or 2H B (bf16); read the
              token's k slots (4 B per pair).
    combine:  per pair read one expert-output row (2H B; with FP8 expert
              outputs H B of codes and 4*H/128 B of scales), its weight and
              slot (8 B); per token write one bf16 row (2H B).
    """
    P = T * k
    layout = 8 * P + 4 * P + 4 * (E + (E + 1) + G)
    row = H + 4 * (H // 128) if fp8 else 2 * H
    dispatch = 2 * H * T + row * R_used + 4 * P
    in_row = H + 4 * (H // 128) if fp8_combine else 2 * H
    combine = in_row * R_used + 8 * P + 2 * H * T
    return dict(layout=layout, dispatch=dispatch, combine=combine)


def ideal_bytes_dedup(T: int, H: int, G: int, k: int, kg: int, used: int, fp8: bool) -> dict:
    """Algorithmic HBM bytes of one pass of the per-group dedup variant, with
    `used` receive rows (one per token and group it reaches).

    layout:   read topk_idx and topk_weights (12 B per pair), write the group
              rows (4 B per entry) and each used row's masked top-k ids and
              weights (12 B per row and k), plus counts and offsets.
    dispatch: read x once (2H B per token) and the entries' rows (4 B each);
              write one receive row per used row (H + 4*H/128 B FP8, 2H bf16).
    combine:  read one bf16 row per used row and the entries' rows (4 B
              each); write one bf16 row per token.
    """
    P = T * k
    layout = 12 * P + 4 * T * kg + 12 * used * k + 4 * (3 * G + 1)
    row = H + 4 * (H // 128) if fp8 else 2 * H
    dispatch = 2 * H * T + 4 * T * kg + row * used
    combine = 2 * H * used + 4 * T * kg + 2 * H * T
    return dict(layout=layout, dispatch=dispatch, combine=combine)


def sources_digest() -> str:
    """Digest of every source of libep.so (kernels, launchers and the C ABI):
    a committed profile counts only while this matches."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def _committed_json(fname: str, tag: str, digest: str):
    """The machine-readable `tag: {...}` line of a committed rocprofv3 summary
    under profiles/, if it was taken on the current kernel sources; else None."""
    path = os.path.join(PROFILES, fname)
    if not os.path.exists(path):
        return None
    m = re.search(tag + r":\s*(\{.*\})", open(path).read())
    if not m:
        return None
    rec = json.loads(m.group(1))
    return rec if rec.get("sources_digest") == digest else None


def committed_traffic(workload: str, digest: str):
    """HBM bytes per launch of each kernel (FETCH_SIZE + WRITE_SIZE, calibrated)
    from profiles/<workload>_traffic.md."""
    return _committed_json("%s_traffic.md" % workload, "traffic_json", digest)


def committed_trace(workload: str, digest: str):
    """Mean kernel durations (us) from profiles/<workload>_kernel_trace.md."""
    return _committed_json("%s_kernel_trace.md" % workload, "trace_json", digest)


def cpu_baseline(wl) -> dict:
    """The oracle as it stands, on this host, over the whole workload: layout +
    FP8 dispatch + combine (the identity expert between them, the oracle's own
    dequantisation, is untimed, like on the GPU).  Timed single-threaded, then
    with the tokens cut into one contiguous range per thread (as many threads
    as the cores this process may run on, capped by the host's OMP_NUM_THREADS
    share); the layout stays one sequential pass, its order being the
    definition.  Each oracle call is single-threaded C that releases the GIL."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    oracle.lib()
    affinity = len(os.sched_getaffinity(0))
    share = int(os.environ.get("OMP_NUM_THREADS") or affinity)
    threads = max(1, min(affinity, share))
    T, H, R = wl.T, wl.H, wl.R

    t0 = time.perf_counter()
    lay = oracle.layout(wl.topk_idx, wl.E, wl.G, wl.cap, want_recv_src=False)
    q, s = oracle.dispatch_fp8(wl.x_bits, lay["slot_idx"], R)
    t1 = time.perf_counter()
    y = oracle.dequant_fp8(q, s)
    del q, s
    t2 = time.perf_counter()
    out1 = oracle.combine(y, wl.topk_weights, lay["slot_idx"])
    t3 = time.perf_counter()
    single = (t1 - t0) + (t3 - t2)

    bounds = np.linspace(0, T, threads + 1).astype(np.int64)
    parts = [(int(bounds[i]), int(bounds[i + 1])) for i in range(threads) if bounds[i + 1] > bounds[i]]
    x, w = wl.x_bits, wl.topk_weights
    with ThreadPoolExecutor(threads) as ex:
        t0 = time.perf_counter()
        lay2 = oracle.layout(wl.topk_idx, wl.E, wl.G, wl.cap, want_recv_src=False)
        sl = lay2["slot_idx"]
        q = np.zeros((R, H), np.uint8)
        s = np.zeros((R, H // 128), np.float32)
        list(ex.map(lambda r: oracle.dispatch_fp8_into(x[r[0]:r[1]], sl[r[0]:r[1]], q, s), parts))
        t1 = time.perf_counter()
        del q, s
        t2 = time.perf_counter()
        out = np.empty((T, H), np.uint16)
        list(ex.map(lambda r: oracle.combine_into(y, w[r[0]:r[1]], sl[r[0]:r[1]], out[r[0]:r[1]]),
                    parts))
        t3 = time.perf_counter()
    multi = (t1 - t0) + (t3 - t2)
    assert (out == out1).all(), "the threaded oracle run must give the single-threaded result"
    used = int((lay["slot_idx"] >= 0).sum())
    b = sum(ideal_bytes(T, H, wl.E, wl.G, wl.k, used, True).values())
    del y, out, out1
    return {"value": round(b / multi / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": "the whole workload (T=%d, H=%d, E=%d, top-%d, FP8 dispatch, bf16 "
                      "combine): layout (one sequential pass) + dispatch + combine, tokens split "
                      "over %d threads, %.3f s; single-threaded %.3f s" % (
                          T, H, wl.E, wl.k, threads, multi, single),
            "seconds": round(multi, 4), "cpu": cpu_model(), "cores_available": affinity,
            "single_thread": {"value": round(b / single / 1e9, 4), "unit": "GB/s", "cores": 1,
                              "seconds": round(single, 4)}}


def cpu_model() -> str:
    """/proc/cpuinfo's model name of the first CPU, with its family, model and
    stepping numbers (a virtual machine may show only the vendor's brand)."""
    fields = {}
    try:
        for ln in open("/proc/cpuinfo"):
            if not ln.strip():
                break
            key, _, val = ln.partition(":")
            fields.setdefault(key.strip(), val.strip())
    except OSError:
        return "unknown"
    name = fields.get("model name", "unknown")
    ids = [(k, fields[k]) for k in ("cpu family", "model", "stepping") if k in fields]
    if ids:
        name += " (%s)" % ", ".join("%s %s" % kv for kv in ids)
    return name


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle timing (profiling runs)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-flush", action="store_true",
                    help="skip the extra steps timed after emptying L2 and the MALL")
    ap.add_argument("--workload", default="dsv3",
                    help="dsv3 (default: the metric's configuration), tiny, skewed, lowlat or large")
    ap.add_argument("--graph", action="store_true",
                    help="record consecutive steps in a HIP graph and time its replays "
                         "(launch-bound workloads); per-kernel times are then not reported")
    ap.add_argument("--graph-steps", type=int, default=10,
                    help="steps recorded in the graph, back to back, as a decode loop's "
                         "layers would be (must divide --steps)")
    ap.add_argument("--pow2", action="store_true",
                    help="FP8 dispatch with power-of-two scales (EP_FP8_E4M3_POW2)")
    ap.add_argument("--fp8-combine", action="store_true",
                    help="expert outputs stay FP8 (the dispatched codes and scales) and combine "
                         "reads them with ep_combine_fp8 (ep_combine_mxfp8 with --mx)")
    ap.add_argument("--fused", action="store_true",
                    help="layout and dispatch through ep_layout_dispatch (one launch for batches "
                         "of at most 4096 pairs); the layout/dispatch split is then not reported")
    ap.add_argument("--read-x-ahead", action="store_true",
                    help="as --fused, with EP_READ_X_AHEAD: the layout launches read x into the "
                         "last-level cache for dispatch")
    ap.add_argument("--mx", action="store_true",
                    help="MXFP8 dispatch (EP_MXFP8_E4M3: one E8M0 scale byte per 32 channels)")
    ap.add_argument("--mn-scales", action="store_true",
                    help="the timed dispatch stores its scales MN-major (EP_SCALES_MN_MAJOR)")
    ap.add_argument("--mn-convert", action="store_true",
                    help="row-major dispatch followed by ep_scales_to_mn_major inside the "
                         "dispatch interval (the conversion's bytes join the dispatch's)")
    ap.add_argument("--f16", action="store_true",
                    help="fp16 path: EP_F16 dispatch and ep_combine_f16 (a bf16 workload's shapes)")
    ap.add_argument("--dedup", action="store_true",
                    help="per-group dedup variant: ep_get_group_layout (with the receiving "
                         "side's metadata), dispatch to the groups, ep_combine_groups")
    args = ap.parse_args()
    if args.read_x_ahead:
        args.fused = True
    if args.dedup and (args.fused or args.fp8_combine or args.f16):
        print("--dedup times its own three calls; it combines with --pow2, --mx and --graph only",
              file=sys.stderr)
        return 2
    if args.mn_convert and (args.mn_scales or args.fused or args.dedup or args.graph):
        print("--mn-convert times layout, dispatch, conversion and combine as separate calls",
              file=sys.stderr)
        return 2
    if args.graph and (args.graph_steps < 1 or args.steps % args.graph_steps != 0):
        print("--graph-steps must be positive and divide --steps", file=sys.stderr)
        return 2
    if args.mn_scales and args.fp8_combine:
        print("--mn-scales does not combine with --fp8-combine (ep_combine_fp8 reads row-major "
              "scales)", file=sys.stderr)
        return 2
    if args.mx and args.pow2:
        print("--mx is its own scale format; it does not combine with --pow2", file=sys.stderr)
        return 2

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the path runs on a single MI355X and has no "
              "multi-GPU mode (asked for --gpus %d)" % args.gpus, file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from combine_moe_layout_amd import binding as B
    from combine_moe_layout_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    name = args.workload
    if name not in W.CONFIGS:
        print("unknown workload %r; choose from %s" % (name, ", ".join(W.CONFIGS)), file=sys.stderr)
        return 2
    wl = W.make(name, seed=args.seed)
    T, H, E, G, k, fp8 = wl.T, wl.H, wl.E, wl.G, wl.k, wl.fp8
    if (args.fp8_combine or args.mx or args.pow2 or args.mn_scales or args.mn_convert) and not fp8:
        print("--fp8-combine, --mx, --pow2, --mn-scales and --mn-convert need an FP8 workload "
              "(dsv3, lowlat, large)",
              file=sys.stderr)
        return 2
    if args.f16:
        fp8 = False  # the fp16 path moves 2-byte rows both ways
    if fp8:
        dtype_enum = B.EP_MXFP8_E4M3 if args.mx else B.EP_FP8_E4M3_POW2 if args.pow2 else B.EP_FP8_E4M3
    else:
        dtype_enum = B.EP_F16 if args.f16 else B.EP_BF16
    # the timed dispatch's dtype; the untimed set-up below writes row-major
    # scales for the identity-expert stand-in
    step_dtype = dtype_enum | (B.EP_SCALES_MN_MAJOR if args.mn_scales else 0)
    if args.read_x_ahead:
        step_dtype |= B.EP_READ_X_AHEAD
    if args.f16:
        # fp16 activations of the same distribution (the bf16 values, converted)
        x = torch.from_numpy(wl.x_bits.view(np.int16)).to(dev).view(torch.bfloat16).to(torch.float16)
    else:
        x = torch.from_numpy(wl.x_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    row_dtype = torch.float16 if args.f16 else torch.bfloat16
    topk_idx = torch.from_numpy(wl.topk_idx).to(dev)
    topk_w = torch.from_numpy(wl.topk_weights).to(dev)
    lay = B.EpLayout(T, k, E, G, wl.cap, device=dev)
    R = lay.num_recv_rows
    if fp8:
        recv_q = torch.empty((R, H), dtype=torch.uint8, device=dev)
        recv_s = (torch.empty((R, H // 32), dtype=torch.uint8, device=dev) if args.mx else
                  torch.empty((R, H // 128), dtype=torch.float32, device=dev))
    else:
        recv_q = torch.empty((R, H), dtype=row_dtype, device=dev)
        recv_s = None
    y = None if args.fp8_combine else torch.empty((R, H), dtype=row_dtype, device=dev)
    out = torch.empty((T, H), dtype=row_dtype, device=dev)

    # identity expert, once, untimed; y is its own buffer, as an expert's output would be
    B.ep_get_layout(topk_idx, lay)
    B.ep_dispatch(x, lay, dtype_enum, recv_q, recv_s)
    if args.fp8_combine:
        pass  # the FP8 receive buffer itself is the expert output
    elif fp8 and args.mx:
        B.ep_dequant_mxfp8(recv_q, recv_s, y)
    elif fp8:
        B.ep_dequant_fp8(recv_q, recv_s, y)
    else:
        B.ep_copy(recv_q, y)
    torch.cuda.synchronize()
    used = int((lay.slot_idx >= 0).sum().item())
    nbytes = ideal_bytes(T, H, E, G, k, used, fp8, args.fp8_combine)
    dedup = None
    if args.dedup:
        # the per-expert buffers above only measure how many rows that path
        # would move; the dedup step has buffers of its own
        del y, recv_q, recv_s
        glay = B.EpGroupLayout(T, k, E, G, device=dev)
        Rg, kg = glay.num_recv_rows, glay.num_topk
        g_ridx = torch.empty((Rg, k), dtype=torch.int64, device=dev)
        g_rw = torch.empty((Rg, k), dtype=torch.float32, device=dev)
        g_q = torch.empty((Rg, H), dtype=torch.uint8 if fp8 else torch.bfloat16, device=dev)
        g_s = None
        if fp8:
            g_s = (torch.empty((Rg, H // 32), dtype=torch.uint8, device=dev) if args.mx else
                   torch.empty((Rg, H // 128), dtype=torch.float32, device=dev))
        g_z = torch.empty((Rg, H), dtype=torch.bfloat16, device=dev)
        B.ep_get_group_layout(topk_idx, topk_w, glay, g_ridx, g_rw)
        B.ep_dispatch(x, glay, dtype_enum, g_q, g_s)
        # identity experts on the receiving side, untimed: one row per (token, group)
        if fp8 and args.mx:
            B.ep_dequant_mxfp8(g_q, g_s, g_z)
        elif fp8:
            B.ep_dequant_fp8(g_q, g_s, g_z)
        else:
            B.ep_copy(g_q, g_z)
        torch.cuda.synchronize()
        g_used = int(glay.expert_offsets[-1].item())
        row_b = H + 4 * (H // 128) if fp8 else 2 * H
        dedup = {"rows": g_used, "rows_per_expert_path": used,
                 "row_ratio": round(g_used / max(used, 1), 4),
                 "dispatch_row_bytes": g_used * row_b, "dispatch_row_bytes_per_expert_path": used * row_b,
                 "combine_row_bytes": g_used * 2 * H, "combine_row_bytes_per_expert_path": used * 2 * H}
        nbytes = ideal_bytes_dedup(T, H, G, k, kg, g_used, fp8)
    recv_s_mn = None
    if args.mn_convert:
        recv_s_mn = torch.empty(tuple(reversed(recv_s.shape)), dtype=recv_s.dtype, device=dev)
        # every row's scales read once and written once
        nbytes["scales_mn"] = 2 * R * (H // 128) * 4
    step_bytes = sum(nbytes.values())

    def step(ev=None, s=None, read_ahead=False):
        # s: the stream to launch on (None = torch's current stream, which is
        # the capture stream while a graph is being recorded).  read_ahead:
        # layout + dispatch through ep_layout_dispatch with EP_READ_X_AHEAD.
        if ev is not None:
            ev[0].record(s)
        if args.dedup:
            B.ep_get_group_layout(topk_idx, topk_w, glay, g_ridx, g_rw, s)
            if ev is not None:
                ev[1].record(s)
            B.ep_dispatch(x, glay, step_dtype, g_q, g_s, s)
            if ev is not None:
                ev[2].record(s)
            B.ep_combine_groups(g_z, glay, out, s)
            if ev is not None:
                ev[3].record(s)
            return
        if args.fused or read_ahead:
            dt = step_dtype | (B.EP_READ_X_AHEAD if read_ahead else 0)
            B.ep_layout_dispatch(topk_idx, lay, x, dt, recv_q, recv_s, s)
            if ev is not None:
                ev[1].record(s)
        else:
            B.ep_get_layout(topk_idx, lay, s)
            if ev is not None:
                ev[1].record(s)
            B.ep_dispatch(x, lay, step_dtype, recv_q, recv_s, s)
            if recv_s_mn is not None:
                B.ep_scales_to_mn_major(recv_s, H, dtype_enum, recv_s_mn, s)
        if ev is not None:
            ev[2].record(s)
        if args.fp8_combine and args.mx:
            B.ep_combine_mxfp8(recv_q, recv_s, topk_w, lay, out, s)
        elif args.fp8_combine:
            B.ep_combine_fp8(recv_q, recv_s, topk_w, lay, out, s)
        elif args.f16:
            B.ep_combine_f16(y, topk_w, lay, out, s)
        else:
            B.ep_combine(y, topk_w, lay, out, s)
        if ev is not None:
            ev[3].record(s)

    for _ in range(args.warmup):
        step(s=stream)
    torch.cuda.synchronize()

    graph = None
    gs = args.graph_steps if args.graph else 1   # steps per replay
    if args.graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(gs):
                step()
        for _ in range(max(1, args.warmup // gs)):
            graph.replay()
        torch.cuda.synchronize()

    # Per-kernel pass: K steps with HIP events recorded around every call on
    # the stream the kernels run on.  The events measure each kernel's own
    # duration (the per-kernel breakdown and the roofline come from here), but
    # each costs a few us of its own on the GPU, so the step rate is taken
    # from the timed loop below, which records none.
    if graph is not None:
        events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)]
                  for _ in range(args.steps // gs)]
    else:
        events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    e0 = time.perf_counter()
    for i in range(len(events)):
        if graph is not None:
            events[i][0].record(stream)
            graph.replay()
            events[i][1].record(stream)
        else:
            step(events[i], stream)
    torch.cuda.synchronize()
    ms_with_events = (time.perf_counter() - e0) * 1e3 / args.steps

    # timed region: exactly K steps, synchronised on both sides, nothing else
    # enqueued between them
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if graph is not None:
        for _ in range(args.steps // gs):
            graph.replay()
    else:
        for _ in range(args.steps):
            step(None, stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    if graph is not None:
        per = {"graph_step": [ev[0].elapsed_time(ev[1]) / gs for ev in events]}
    elif args.fused:
        per = {"layout_dispatch": [ev[0].elapsed_time(ev[2]) for ev in events]}
    else:
        per = {"layout": [ev[0].elapsed_time(ev[1]) for ev in events],
               "dispatch": [ev[1].elapsed_time(ev[2]) for ev in events]}
    if graph is None:
        per["combine"] = [ev[2].elapsed_time(ev[3]) for ev in events]
    us = {kname: float(np.mean(v)) * 1e3 for kname, v in per.items()}
    p50 = {kname: float(np.percentile(v, 50)) * 1e3 for kname, v in per.items()}
    p95 = {kname: float(np.percentile(v, 95)) * 1e3 for kname, v in per.items()}
    p99 = {kname: float(np.percentile(v, 99)) * 1e3 for kname, v in per.items()}

    # The same step with the caches emptied first: before each of these steps a
    # 512 MiB buffer (twice the 256 MB MALL) is read, outside the events, so
    # nothing of the previous step is left in L2 or the MALL and the dirty
    # lines it left are written back before the step starts.  (Writing the
    # buffer instead would leave the MALL full of dirty lines whose write-back
    # the next step's writes would pay for.)  Three passes: events around every
    # call (per-kernel times); events only at the step's two ends (the step's
    # own time, with no event inside it); and, where it applies, the step with
    # layout + dispatch through ep_layout_dispatch with EP_READ_X_AHEAD.  The
    # timed loop above is the steady state.
    flushed = None
    read_ahead_applies = not (args.dedup or args.fused or args.mn_convert) and T * k > 4096
    if graph is None and not args.no_flush:
        flush_buf = torch.zeros((512 << 20) // 8, dtype=torch.int64, device=dev)
        n_flush = min(args.steps, 50)

        def flushed_pass(n_events, read_ahead=False):
            evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n_flush)]
            for i in range(n_flush):
                flush_buf.sum()
                if n_events == 4:
                    step(evs[i], stream, read_ahead)
                else:
                    evs[i][0].record(stream)
                    step(None, stream, read_ahead)
                    evs[i][3].record(stream)
            torch.cuda.synchronize()
            return evs

        fev = flushed_pass(4)
        first = "layout_dispatch" if args.fused else "layout"
        fper = {first: [ev[0].elapsed_time(ev[1]) for ev in fev]}
        if not args.fused:
            fper["dispatch"] = [ev[1].elapsed_time(ev[2]) for ev in fev]
        fper["combine"] = [ev[2].elapsed_time(ev[3]) for ev in fev]
        flushed = {"kernel_us_mean": {kname: round(float(np.mean(v)) * 1e3, 2) for kname, v in fper.items()}}
        whole = [ev[0].elapsed_time(ev[3]) * 1e3 for ev in flushed_pass(2)]
        flushed["step_us"] = round(float(np.mean(whole)), 2)
        flushed["step_us_p50"] = round(float(np.percentile(whole, 50)), 2)
        if read_ahead_applies:
            rev = flushed_pass(4, read_ahead=True)
            whole_ra = [ev[0].elapsed_time(ev[3]) * 1e3 for ev in flushed_pass(2, read_ahead=True)]
            flushed["read_x_ahead"] = {
                "kernel_us_mean": {
                    "layout_dispatch": round(float(np.mean([e[0].elapsed_time(e[1]) for e in rev])) * 1e3, 2),
                    "combine": round(float(np.mean([e[2].elapsed_time(e[3]) for e in rev])) * 1e3, 2)},
                "step_us": round(float(np.mean(whole_ra)), 2),
                "step_us_p50": round(float(np.percentile(whole_ra, 50)), 2)}
        del flush_buf

    # the steady state of the read-ahead form (x already cached when it runs)
    steady_read_ahead = None
    if graph is None and read_ahead_applies:
        for _ in range(3):
            step(None, stream, True)
        torch.cuda.synchronize()
        r0 = time.perf_counter()
        for _ in range(args.steps):
            step(None, stream, True)
        torch.cuda.synchronize()
        steady_read_ahead = (time.perf_counter() - r0) * 1e6 / args.steps

    # plain copy of the same size as combine's traffic: the practical ceiling
    copy_bytes = 1 << 30
    src = torch.empty(copy_bytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        B.ep_copy(src, dst, stream)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    reps = 10
    for _ in range(reps):
        B.ep_copy(src, dst, stream)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 2 * copy_bytes * reps / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del src, dst

    # the scale-layout conversion alone (its share of the dispatch interval)
    convert = None
    if recv_s_mn is not None:
        c0.record(stream)
        for _ in range(50):
            B.ep_scales_to_mn_major(recv_s, H, dtype_enum, recv_s_mn, stream)
        c1.record(stream)
        torch.cuda.synchronize()
        conv_us = c0.elapsed_time(c1) * 1e3 / 50
        convert = {"us": round(conv_us, 2), "bytes": nbytes["scales_mn"],
                   "gbps": round(nbytes["scales_mn"] / (conv_us * 1e-6) / 1e9, 1)}

    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    if graph is None:
        t_dispatch = us["layout_dispatch"] if args.fused else us["dispatch"]
        d_bytes = nbytes["dispatch"] + (nbytes["layout"] if args.fused else 0) + nbytes.get("scales_mn", 0)
        dc_gbps = (d_bytes + nbytes["combine"]) / ((t_dispatch + us["combine"]) * 1e-6) / 1e9
        combine_gbps = nbytes["combine"] / (us["combine"] * 1e-6) / 1e9
        dispatch_gbps = d_bytes / (t_dispatch * 1e-6) / 1e9
    else:
        dc_gbps = combine_gbps = dispatch_gbps = None
    digest = sources_digest()
    # the committed summaries: HBM traffic (two counter runs) and kernel-trace
    # means of the default step of each workload, valid on the current sources
    default_path = not (args.dedup or args.mx or args.f16 or args.pow2 or args.fp8_combine
                        or args.mn_scales or args.mn_convert or args.fused)
    traffic = committed_traffic(name, digest) if default_path else None
    trace = committed_trace(name, digest) if default_path else None

    result = {
        "metric": "dispatch+combine effective HBM GB/s (% peak) at 8K tok×7168, top-8/256",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic (seeded: x ~ N(0,1) bf16; routing %s)" % W.CONFIGS[name][7],
        "config": {"workload": W.DESCRIPTIONS[name], "name": name, "T": T, "hidden": H,
                   "experts": E, "groups": G, "topk": k, "capacity": wl.cap,
                   "dispatch_dtype": ("mxfp8 (e4m3+e8m0 scale/32ch)" if args.mx else
                                      "fp8_e4m3+pow2 scale/128ch" if args.pow2 else
                                      "fp8_e4m3+fp32 scale/128ch") +
                                     (", scales MN-major" if args.mn_scales else
                                      ", then scales converted to MN-major" if args.mn_convert
                                      else "") if fp8 else
                                     "fp16" if args.f16 else "bf16",
                   "combine_dtype": ("mxfp8 in, bf16 out" if args.mx else "fp8_e4m3 in, bf16 out")
                   if args.fp8_combine else
                                    "fp16" if args.f16 else "bf16",
                   "step": "group_layout+dispatch_to_groups+combine_groups (per-group dedup)"
                   if args.dedup else "layout_dispatch (fused call)+combine" if args.fused
                   else "layout+dispatch+combine"},
        "pct_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "ms_per_step_with_events": round(ms_with_events, 5),
        "ideal_bytes": nbytes,
        "kernel_us_mean": {kk: round(v, 2) for kk, v in us.items()},
        "kernel_us_p50": {kk: round(v, 2) for kk, v in p50.items()},
        "kernel_us_p95": {kk: round(v, 2) for kk, v in p95.items()},
        "kernel_us_p99": {kk: round(v, 2) for kk, v in p99.items()},
        "caches": "value and kernel_us_*: steps back to back (x stays in the MALL between "
                  "steps); after_flush: each step after a 512 MiB read empties L2 and the MALL",
        "copy_kernel_gbps": round(copy_gbps, 1),
        "sources_digest": digest,
    }
    if graph is None:
        result["dispatch_plus_combine_gbps"] = round(dc_gbps, 1)
        result["dispatch_plus_combine_pct_peak"] = round(100 * dc_gbps / HBM_PEAK_GBPS, 2)
        result["dispatch_gbps"] = round(dispatch_gbps, 1)
        roof = {
            "kernel": "combine_groups" if args.dedup else
            ("combine_mxfp8" if args.mx else "combine_fp8") if args.fp8_combine
            else "combine_f16" if args.f16 else "combine", "bound": "hbm",
            "achieved": round(combine_gbps, 1),
            "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(combine_gbps / HBM_PEAK_GBPS, 4),
            "traffic": None if traffic is None else traffic["bytes_per_launch"]["combine"],
            "algorithmic_bytes": nbytes["combine"],
            "time_source": "mean of HIP events recorded just before and after each combine launch "
                           "on its stream, over the %d steps of the per-kernel pass; each interval "
                           "also holds the events' own cost (a few us)" % args.steps,
            "launch_us": round(us["combine"], 2)}
        if trace is not None:
            # the committed rocprofv3 kernel trace (kernel start to end, no events)
            t_c = trace["avg_us"]["combine"]
            roof["profile_launch_us"] = t_c
            roof["profile_frac"] = round(nbytes["combine"] / (t_c * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)
            roof["profile"] = "profiles/%s_kernel_trace.md" % name
            # every kernel of the step as the committed trace timed it, and
            # dispatch + combine over those times
            avg = trace["avg_us"]
            layout_us = sum(v for kk, v in avg.items() if kk.startswith("layout"))
            result["kernel_us_profile"] = {"layout": round(layout_us, 2),
                                           "dispatch": avg.get("dispatch"), "combine": t_c,
                                           "source": roof["profile"]}
            if "dispatch" in avg:
                dc_p = (nbytes["dispatch"] + nbytes["combine"]) / ((avg["dispatch"] + t_c) * 1e-6) / 1e9
                result["kernel_us_profile"]["dispatch_plus_combine_pct_peak"] = round(
                    100 * dc_p / HBM_PEAK_GBPS, 2)
        result["roofline"] = roof
    else:
        result["config"]["step"] += " (HIP graph replay, %d steps per graph)" % gs
        result["graph_steps"] = gs
    if flushed is not None:
        d_key = "layout_dispatch" if args.fused else "dispatch"
        d_bytes_f = nbytes["dispatch"] + (nbytes["layout"] if args.fused else 0) + nbytes.get("scales_mn", 0)
        fk = flushed["kernel_us_mean"]
        dc_f = (d_bytes_f + nbytes["combine"]) / ((fk[d_key] + fk["combine"]) * 1e-6) / 1e9
        flushed["dispatch_plus_combine_gbps"] = round(dc_f, 1)
        flushed["dispatch_plus_combine_pct_peak"] = round(100 * dc_f / HBM_PEAK_GBPS, 2)
        flushed["dispatch_roofline_frac"] = round(
            d_bytes_f / (fk[d_key] * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)
        # whole step, events at its ends only: all the step's bytes, and the
        # dispatch + combine bytes alone (the layout's time stays in the denominator)
        for key, form in ((None, flushed), ("read_x_ahead", flushed.get("read_x_ahead"))):
            if form is None:
                continue
            st_us = form["step_us"]
            form["step_gbps"] = round(step_bytes / (st_us * 1e-6) / 1e9, 1)
            form["step_pct_peak"] = round(100 * step_bytes / (st_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 2)
            dc_b = step_bytes - nbytes["layout"]
            form["dispatch_plus_combine_pct_peak_of_step"] = round(
                100 * dc_b / (st_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 2)
        result["after_flush"] = flushed
        # the earlier names of two of these figures
        result["kernel_us_mean_after_flush"] = fk
        result["dispatch_plus_combine_gbps_after_flush"] = round(dc_f, 1)
    if steady_read_ahead is not None:
        result["read_x_ahead_steady_step_us"] = round(steady_read_ahead, 2)
    if dedup is not None:
        result["dedup"] = dedup
    if convert is not None:
        result["scales_mn_conversion"] = convert
    if not args.no_cpu_baseline and name == "dsv3" and default_path:
        result["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

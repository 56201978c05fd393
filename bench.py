"""Benchmark of the MoE expert-parallel hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input that
is already resident in HBM: route (top-k gating) -> dispatch layout ->
dispatch -> combine, on the DeepSeek-V3-like workload (T=4096 tokens,
H=7168 bf16, E=256 experts over R=32 virtual ranks, top-8) -- one EP rank's
share of the EP=32, 4096-token, H=7168, top-8 dispatch/combine benchmark.
The fused flag-in-payload mode and the backward pass (combine_grad ->
dispatch_grad) are timed beside it on the same inputs.

Prints ONE JSON line.  `value` = algorithmic HBM bytes of a whole step /
step time (GB/s); tokens/s and the fraction of the 8 TB/s HBM peak ride along.
`roofline` is measured live: every op of every timed step records a
hipEvent_t from its own last kernel's dispatch packet (the library's timing
hook, no marker packet), on the stream it runs on; an op's duration is the
interval from the previous op's end to its own end, which for these
back-to-back kernels is the kernel time a trace profiler reports.
`cpu_baseline` times the CPU oracle on this host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "dispatch+combine effective HBM GB/s (% of MI355X peak) and tokens/s"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="dsv3")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fused", action="store_true")
    ap.add_argument("--no-fused-incast", action="store_true",
                    help="skip the fused mode on the skewed incast workload")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the forward step (and fused call) on the other workloads")
    ap.add_argument("--no-pipelined", action="store_true")
    ap.add_argument("--no-coalesce", action="store_true",
                    help="skip the rank-coalesced send leg (one record per token and rank)")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the leg that replays the step from a captured HIP graph")
    ap.add_argument("--fused-modes", default="0,1,2,3,4",
                    help="comma-separated fused synchronisation modes to time")
    ap.add_argument("--partition-sweep", action="store_true",
                    help="instead of the step: the window-copy consumer under per-peer, "
                         "equal-slice and LPT schedules (one JSON line)")
    ap.add_argument("--sync-sweep", action="store_true",
                    help="instead of the step: the fused mode's synchronisation variants "
                         "against three launches, over the row size (one JSON line)")
    ap.add_argument("--no-isolated", action="store_true",
                    help="skip the per-op timings after a cache-clearing overwrite")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 512 MiB device-to-device copy --steps times "
                         "(scales the HBM byte counters of a profiler run)")
    return ap.parse_args()


def copy_calibration(steps: int) -> None:
    import torch
    n = 512 << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / steps
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "steps": steps,
                      "us_per_copy": round(us, 2), "gbps": round(2 * n / us / 1e3, 1)}),
          flush=True)


# Source files whose text determines each kernel's memory traffic.
KERNEL_SOURCES = {
    "dispatch": ["dispatch.hip", "ep_device.h", "ep_internal.h"],
    "combine": ["combine.hip", "ep_combine_dev.h", "ep_device.h", "ep_internal.h"],
    "combine_grad": ["backward.hip", "ep_combine_dev.h", "ep_device.h", "ep_internal.h"],
    "dispatch_grad": ["combine.hip", "ep_combine_dev.h", "ep_device.h", "ep_internal.h"],
    "fused": ["fused.hip", "ep_combine_dev.h", "ep_device.h", "ep_internal.h", "ep_layout_dev.h"],
}


def src_digest(names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "combine_ep_route_topk_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, or None
    when absent or when the kernel's sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as f:
        for ln in f:
            if ln.startswith("json:"):
                rec = json.loads(ln[5:])
    if rec.get("source_sha256_16") != src_digest(KERNEL_SOURCES[kernel]):
        return None
    return rec.get("hbm_bytes_per_launch")


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.steps)
        return
    if args.sync_sweep and args.gpus == 1:
        sync_sweep(args)
        return
    if args.partition_sweep and args.gpus == 1:
        partition_sweep(args)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the multi-GPU "
                                   "exchange is not part of it; run with --gpus 1"}))
        sys.exit(2)

    import torch

    from combine_ep_route_topk_amd import ep
    from combine_ep_route_topk_amd import workloads as wl

    dev = torch.device("cuda:0")
    w = wl.WORKLOADS[args.workload]
    T, H, E, R, k = w.T, w.H, w.E, w.R, w.k
    inp = wl.make_inputs(w)
    logits = torch.from_numpy(inp["logits"]).to(dev)
    x = torch.from_numpy(inp["x"].view(np.int16)).to(dev).view(torch.bfloat16)

    # pre-allocated outputs: the timed region allocates nothing
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    wt = torch.empty((T, k), dtype=torch.float32, device=dev)
    lay = ep.layout_outputs(T, k, E, R, dev, slot_src=True)
    send = torch.empty((T * k, H), dtype=torch.bfloat16, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)

    hip = ep.HipEvents()
    # Validated once, then each step is four bare C calls (the per-call tensor
    # checks of the convenience wrappers cost more host time than the kernels).
    ops = [ep.bind_route_topk(logits, k, True, idx, wt, stream),
           ep.bind_dispatch_layout(idx, E, R, lay, stream),
           ep.bind_dispatch(x, lay["pos"], send, stream),
           ep.bind_combine(send, lay["pos"], wt, out, stream)]
    set_events = ep.library().ep_set_timing_events

    step = make_step(ops, set_events)

    # correctness gate before timing: the identity-expert round trip is exact
    step()
    torch.cuda.synchronize()
    if not torch.equal(out.view(torch.int16), x.view(torch.int16)):
        print(json.dumps({"error": "parity gate failed: combine(dispatch(x)) != x"}))
        sys.exit(1)
    if ep.ep_get_device_error(lay["workspace"]) != ep.EP_OK:
        print(json.dumps({"error": "layout reported a device error"}))
        sys.exit(1)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    names = ["route", "layout", "dispatch", "combine"]
    per_op, wall = time_steps(torch, hip, step, names, K)
    mean_us = {n: float(np.mean(v)) for n, v in per_op.items()}
    p10_us = {n: float(np.percentile(v, 10)) for n, v in per_op.items()}
    p90_us = {n: float(np.percentile(v, 90)) for n, v in per_op.items()}

    ab = wl.algorithmic_bytes(w)
    step_bytes = sum(ab.values())
    ms_per_step = wall / K * 1e3
    step_gbps = step_bytes / (ms_per_step * 1e-3) / 1e9
    # the metric: dispatch + combine algorithmic bytes over their own time
    dc_us = mean_us["dispatch"] + mean_us["combine"]
    dc_bytes = ab["dispatch"] + ab["combine"]
    value = dc_bytes / (dc_us * 1e-6) / 1e9

    dom = "dispatch" if mean_us["dispatch"] >= mean_us["combine"] else "combine"
    achieved = ab[dom] / (mean_us[dom] * 1e-6) / 1e9
    roofline = {
        "kernel": dom,
        "bound": "hbm",
        "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBPS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBPS, 4),
        "traffic": traffic_for(dom, w.name),
        "algorithmic_bytes_per_launch": ab[dom],
        "avg_launch_us": round(mean_us[dom], 2),
    }

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.describe(), "global_batch": T, "hidden": H,
                   "experts": E, "virtual_ranks": R, "top_k": k,
                   "step": "route -> layout -> dispatch -> combine"},
        "value_is": "(dispatch + combine algorithmic bytes) / (dispatch time + combine time), "
                    "per-op times from the ops' own kernels inside back-to-back steps: x stays "
                    "in the Infinity Cache between steps, and dispatch leaves the rows of its "
                    "last tokens (up to 128 MiB) there for combine; isolated_dispatch_combine "
                    "reads every input from HBM",
        "tokens_per_s": round(T / (dc_us * 1e-6), 1),
        "pct_of_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "dispatch_combine_us": round(dc_us, 2),
        "step": {"us": round(ms_per_step * 1e3, 2), "gbps": round(step_gbps, 1),
                 "pct_of_peak": round(100 * step_gbps / HBM_PEAK_GBPS, 2),
                 "tokens_per_s": round(T / (ms_per_step * 1e-3), 1),
                 "what": "route + layout + dispatch + combine, all four ops' algorithmic bytes "
                         "over the wall time per step (= ms_per_step)"},
        "per_op_us": {n: round(v, 2) for n, v in mean_us.items()},
        "per_op_p10_p90_us": {n: [round(p10_us[n], 2), round(p90_us[n], 2)] for n in names},
        # a timing is taken as stable when p90 / p10 <= 1.2 (RailWave's rule)
        "per_op_p90_over_p10": {n: round(p90_us[n] / p10_us[n], 3) for n in names},
        "algorithmic_bytes": ab,
        "roofline": roofline,
    }

    result["copy_achievable"] = copy_achievable(torch, dev, stream)

    if not args.no_isolated:
        iso = bench_isolated(ep, torch, hip, ops, names, set_events, dev, stream)
        result["isolated"] = iso
        iso_us = iso["dispatch"]["median_us"] + iso["combine"]["median_us"]
        result["isolated_dispatch_combine"] = {
            "us": round(iso_us, 2), "gbps": round(dc_bytes / (iso_us * 1e-6) / 1e9, 1),
            "pct_of_peak": round(100 * dc_bytes / (iso_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 2),
            "what": "the metric with each op's inputs read from HBM (each op runs after a "
                    "1 GiB read); value is the back-to-back step, where x stays cached"}

    if not args.no_pipelined:
        ms_p, ok_p, enq_p = bench_pipelined(ep, torch, w, logits, x, dev, K, args.warmup)
        result["pipelined"] = {
            "ms_per_step": round(ms_p, 4),
            "host_enqueue_ms_per_step": round(enq_p, 4),
            "value": round(step_bytes / (ms_p * 1e-3) / 1e9, 1) if ok_p else None,
            "tokens_per_s": round(T / (ms_p * 1e-3), 1) if ok_p else None,
            "parity": ok_p,
            "what": "route + layout of the next batch on a second stream during this batch's "
                    "dispatch and combine; every step still runs all four ops"}

    if not args.no_graph:
        ms_g, ok_g = bench_graph(ep, torch, w, logits, x, dev, K, args.warmup)
        result["graph"] = {
            "ms_per_step": round(ms_g, 4),
            "value": round(step_bytes / (ms_g * 1e-3) / 1e9, 1) if ok_g else None,
            "tokens_per_s": round(T / (ms_g * 1e-3), 1) if ok_g else None,
            "parity": ok_g,
            "steps_per_graph": GRAPH_STEPS,
            "what": "steps captured in a HIP graph and replayed: the same kernels, one graph "
                    "launch per steps_per_graph steps instead of four entry-point calls per step"}

    if not args.no_coalesce and w.E // w.R <= 64:
        result["coalesce"] = bench_coalesce(ep, torch, w, idx, x, dev, K)

    if not args.no_fused:
        result["fused"] = bench_fused(ep, torch, w, x, idx, wt, stream, K, args.warmup,
                                      tuple(int(m) for m in args.fused_modes.split(",") if m))
        if w.name != "incast" and not args.no_fused_incast:
            result["fused_incast"] = bench_fused_workload(ep, torch, wl.WORKLOADS["incast"], dev,
                                                          stream, args.warmup)

    if not args.no_workloads:
        result["workloads"] = bench_workloads(ep, torch, hip, set_events, dev, stream,
                                              [n for n in ("decode", "glm45air", "incast")
                                               if n != w.name], args.warmup)
    if not args.no_backward:
        result["backward"] = bench_backward(ep, torch, hip, set_events, w, x, lay, wt, send,
                                            dev, stream, K, args.warmup, not args.no_isolated)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, inp, lay, args.cpu_seconds, step_bytes)

    print(json.dumps(result), flush=True)


def bench_pipelined(ep, torch, w, logits, x, dev, K, W):
    """Steps whose preprocessing is pipelined (UBEP sec. 5.2: the
    preprocessing steps are pipelined with the transfers): route and layout of
    batch i+1 run on a second stream while batch i's dispatch runs -- dispatch
    fills only five eighths of the CUs -- and its combine.  Every step still runs all four
    ops on its own batch; routing and layout outputs are double-buffered, and
    stream events order each buffer's reuse.  Returns the wall time per step
    and the parity of every step's output."""
    T, H, E, R, k = w.T, w.H, w.E, w.R, w.k
    s0 = torch.cuda.current_stream(dev)
    s1 = torch.cuda.Stream(device=dev)             # default priority
    buf = []
    for _ in range(2):
        b = {"idx": torch.empty((T, k), dtype=torch.int32, device=dev),
             "wt": torch.empty((T, k), dtype=torch.float32, device=dev),
             "lay": ep.layout_outputs(T, k, E, R, dev, slot_src=True)}
        buf.append(b)
    send = torch.empty((T * k, H), dtype=torch.bfloat16, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    pre = [[ep.bind_route_topk(logits, k, True, b["idx"], b["wt"], s1),
            ep.bind_dispatch_layout(b["idx"], E, R, b["lay"], s1)] for b in buf]
    post = [[ep.bind_dispatch(x, b["lay"]["pos"], send, s0),
             ep.bind_combine(send, b["lay"]["pos"], b["wt"], out, s0)] for b in buf]

    def run(n):
        lay_done = [torch.cuda.Event(), torch.cuda.Event()]
        comb_done = [torch.cuda.Event(), torch.cuda.Event()]
        s1.wait_stream(s0)
        for op in pre[0]:
            op()
        lay_done[0].record(s1)
        for i in range(n):
            b = i % 2
            s0.wait_event(lay_done[b])
            for op in post[b]:
                op()
            comb_done[b].record(s0)
            if i + 1 < n:
                nb = (i + 1) % 2
                if i >= 1:
                    s1.wait_event(comb_done[nb])     # batch i-1 no longer reads buffer nb
                for op in pre[nb]:
                    op()
                lay_done[nb].record(s1)
        s0.wait_stream(s1)

    run(W if W > 1 else 2)
    torch.cuda.synchronize()
    ok = torch.equal(out.view(torch.int16), x.view(torch.int16))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(K)
    t_enq = time.perf_counter() - t0
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ok = ok and torch.equal(out.view(torch.int16), x.view(torch.int16))
    for b in buf:
        ok = ok and ep.ep_get_device_error(b["lay"]["workspace"]) == ep.EP_OK
    return wall / K * 1e3, ok, t_enq / K * 1e3


def bench_coalesce(ep, torch, w, idx, x, dev, K):
    """Rank-level token coalescing (RailWave sec. 3.1-3.2: one send record per
    token and destination rank): ep_rank_coalesce then ep_dispatch with its
    first-pick positions, against ep_dispatch_layout then ep_dispatch.  The
    records replace the T*k per-expert rows a multi-GPU exchange would send.
    Reports both pairs' times (back to back, HIP events on the stream), the
    record count and the parity of the coalesced rows."""
    T, H, E, R, k = w.T, w.H, w.E, w.R, w.k
    s = torch.cuda.current_stream(dev)
    lay = ep.layout_outputs(T, k, E, R, dev, slot_src=False)
    co = ep.coalesce_outputs(T, k, E, R, dev)
    send = torch.empty((T * k, H), dtype=torch.bfloat16, device=dev)

    def timed(fn):
        for _ in range(3):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(s)
        for _ in range(K):
            fn()
        b.record(s)
        b.synchronize()
        return a.elapsed_time(b) * 1e3 / K

    def plain():
        ep.ep_dispatch_layout(idx, E, R, out=lay)
        ep.ep_dispatch(x, lay["pos"], send)

    def coalesced():
        ep.ep_rank_coalesce(idx, E, R, out=co)
        ep.ep_dispatch(x, co["send_pos"], send)

    us_plain = timed(plain)
    us_co = timed(coalesced)
    torch.cuda.synchronize()
    C = int(co["rank_offsets"][R].item())
    src = co["row_src"][:C].long()
    ok = bool(torch.equal(send[:C].view(torch.int16), x[src].view(torch.int16)))
    ok = ok and ep.ep_get_device_error(co["workspace"]) == ep.EP_OK
    return {"records": C, "picks": T * k, "records_per_pick": round(C / (T * k), 4),
            "us_layout_dispatch": round(us_plain, 2), "us_coalesce_dispatch": round(us_co, 2),
            "rows_written_saved_bytes": (T * k - C) * H * 2, "parity": ok,
            "what": "ep_rank_coalesce + ep_dispatch(send_pos) against ep_dispatch_layout + "
                    "ep_dispatch, back to back"}


GRAPH_STEPS = 8


def bench_graph(ep, torch, w, logits, x, dev, K, W):
    """GRAPH_STEPS steps (route -> layout -> dispatch -> combine each) captured
    once in a HIP graph on a side stream and replayed.  The library launches
    only kernels (no memory set or copy nodes, no allocation), so the graph
    holds the eager steps' kernels; one graph launch replaces GRAPH_STEPS x 4
    entry-point calls.  (One step per graph is slower than the eager step on
    MI355X: the graph launch itself costs about what it saves.)  Returns the
    wall time per step over ceil(K / GRAPH_STEPS) replays and the parity of
    the output."""
    T, H, E, R, k = w.T, w.H, w.E, w.R, w.k
    s = torch.cuda.Stream(device=dev)              # default priority
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    wt = torch.empty((T, k), dtype=torch.float32, device=dev)
    lay = ep.layout_outputs(T, k, E, R, dev, slot_src=False)
    send = torch.empty((T * k, H), dtype=torch.bfloat16, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    ops = [ep.bind_route_topk(logits, k, True, idx, wt, s),
           ep.bind_dispatch_layout(idx, E, R, lay, s),
           ep.bind_dispatch(x, lay["pos"], send, s),
           ep.bind_combine(send, lay["pos"], wt, out, s)]
    s.wait_stream(torch.cuda.current_stream(dev))
    for _ in range(2):                             # eager warm-up on the capture stream
        for op in ops:
            op()
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for _ in range(GRAPH_STEPS):
            for op in ops:
                op()
    out.fill_(0)
    torch.cuda.synchronize()
    for _ in range(max(W // GRAPH_STEPS, 1)):
        g.replay()
    torch.cuda.synchronize()
    ok = torch.equal(out.view(torch.int16), x.view(torch.int16))
    reps = max(-(-K // GRAPH_STEPS), 1)
    t0 = time.perf_counter()
    for _ in range(reps):
        g.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ok = ok and torch.equal(out.view(torch.int16), x.view(torch.int16))
    ok = ok and ep.ep_get_device_error(lay["workspace"]) == ep.EP_OK
    del g
    return wall / (reps * GRAPH_STEPS) * 1e3, ok


def make_step(ops, set_events):
    def step(stops=None, first_start=None):
        # stops[i]: hipEvent_t recorded by op i's own last kernel (library
        # timing hook); only the region's very first op also records a start.
        for i, op in enumerate(ops):
            if stops is not None:
                set_events(first_start if i == 0 else None, stops[i])
            op()
    return step


def time_steps(torch, hip, step, names, K):
    """K timed steps; returns (per-op durations in us, wall seconds).  Op i of
    step s spans from the end of the op before it (back-to-back kernels on one
    stream) to the end of its own last kernel."""
    stops = [[hip.create() for _ in names] for _ in range(K)]
    region_start = hip.create()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(stops[i], region_start if i == 0 else None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_op = {n: [] for n in names}
    prev = region_start
    for s_ev in stops:
        for j, n in enumerate(names):
            per_op[n].append(hip.elapsed_ms(prev, s_ev[j]) * 1e3)
            prev = s_ev[j]
    for s_ev in stops:
        for e in s_ev:
            hip.destroy(e)
    hip.destroy(region_start)
    return per_op, wall


def bench_workloads(ep, torch, hip, set_events, dev, stream, names, W, K=20):
    """The forward step (route -> layout -> dispatch -> combine) on each other
    workload, timed like the headline (each op's own kernels, back to back),
    behind the same parity gate; and the fused call (item events) where the
    fused leg does not already cover the workload."""
    from combine_ep_route_topk_amd import workloads as wl
    out = {}
    for name in names:
        w = wl.WORKLOADS[name]
        T, H, E, R, k = w.T, w.H, w.E, w.R, w.k
        inp = wl.make_inputs(w)
        logits = torch.from_numpy(inp["logits"]).to(dev)
        x = torch.from_numpy(inp["x"].view(np.int16)).to(dev).view(torch.bfloat16)
        del inp
        idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        wt = torch.empty((T, k), dtype=torch.float32, device=dev)
        lay = ep.layout_outputs(T, k, E, R, dev, slot_src=True)
        send = torch.empty((T * k, H), dtype=torch.bfloat16, device=dev)
        y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        ops = [ep.bind_route_topk(logits, k, True, idx, wt, stream),
               ep.bind_dispatch_layout(idx, E, R, lay, stream),
               ep.bind_dispatch(x, lay["pos"], send, stream),
               ep.bind_combine(send, lay["pos"], wt, y, stream)]
        step = make_step(ops, set_events)
        step()
        torch.cuda.synchronize()
        if not torch.equal(y.view(torch.int16), x.view(torch.int16)) or \
                ep.ep_get_device_error(lay["workspace"]) != ep.EP_OK:
            out[name] = {"workload": w.describe(), "status": "parity gate failed"}
            continue
        for _ in range(W):
            step()
        names4 = ["route", "layout", "dispatch", "combine"]
        per_op, wall = time_steps(torch, hip, step, names4, K)
        mean_us = {n: float(np.mean(v)) for n, v in per_op.items()}
        ab = wl.algorithmic_bytes(w)
        dc_us = mean_us["dispatch"] + mean_us["combine"]
        gbps = (ab["dispatch"] + ab["combine"]) / (dc_us * 1e-6) / 1e9
        res = {"workload": w.describe(),
               "per_op_us": {n: round(v, 2) for n, v in mean_us.items()},
               "dispatch_combine_us": round(dc_us, 2), "gbps": round(gbps, 1),
               "pct_of_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
               "step_us": round(wall / K * 1e6, 2), "parity": True}
        if name != "incast":
            f = bench_fused(ep, torch, w, x, idx, wt, stream, K, W, modes=(0,))
            res["fused_us"] = f["us_per_call"]
            res["fused_status"] = f["sync_modes"].get("item_events", {}).get("status")
        out[name] = res
        del logits, x, idx, wt, lay, send, y, ops, step
        torch.cuda.empty_cache()
    return out


def bench_backward(ep, torch, hip, set_events, w, x, lay, wt, send, dev, stream, K, W,
                   isolated):
    """The backward pass (HyperParallel-MoE sec. 2.2, Fig. 2(b)) on the same
    workload with identity experts: combine_grad(grad_out = x, y = send) then
    dispatch_grad(grad_send = grad_y), back to back on one stream."""
    from combine_ep_route_topk_amd import workloads as wl
    T, H, k = w.T, w.H, w.k
    grad_y = torch.empty((T * k, H), dtype=torch.bfloat16, device=dev)
    grad_w = torch.empty((T, k), dtype=torch.float32, device=dev)
    grad_x = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    ops = [ep.bind_combine_grad(x, send, lay["pos"], wt, grad_y, grad_w, stream),
           ep.bind_dispatch_grad(grad_y, lay["pos"], grad_x, stream)]
    names = ["combine_grad", "dispatch_grad"]
    step = make_step(ops, set_events)
    step()
    torch.cuda.synchronize()
    # gate: identity experts give every pick of a token the same <x_t, x_t>
    if not torch.equal(grad_w, grad_w[:, :1].expand(T, k)):
        return {"status": "parity gate failed: grad_w differs across the picks of a token"}
    ref = x.float().pow(2).sum(dim=1)
    if not torch.allclose(grad_w[:, 0], ref, rtol=1e-4, atol=0.0):
        return {"status": "parity gate failed: grad_w != <x_t, x_t>"}
    for _ in range(W):
        step()
    per_op, wall = time_steps(torch, hip, step, names, K)
    ab = wl.algorithmic_bytes_backward(w)
    res = {}
    for n in names:
        us = float(np.mean(per_op[n]))
        p10, p90 = np.percentile(per_op[n], [10, 90])
        res[n] = {"us": round(us, 2), "gbps": round(ab[n] / (us * 1e-6) / 1e9, 1),
                  "pct_of_peak": round(100 * ab[n] / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 2),
                  "p90_over_p10": round(float(p90 / p10), 3),
                  "algorithmic_bytes": ab[n], "traffic": traffic_for(n, w.name)}
    us_step = wall / K * 1e6
    res["us_per_step"] = round(us_step, 2)
    res["gbps_per_step"] = round(sum(ab.values()) / (us_step * 1e-6) / 1e9, 1)
    if isolated:
        res["isolated"] = bench_isolated(ep, torch, hip, ops, names, set_events, dev, stream)
    res["what"] = "combine_grad -> dispatch_grad, identity experts, back to back"
    del grad_y, grad_w, grad_x
    return res


def copy_achievable(torch, dev, stream, mib=448, reps=20):
    """The "achievable" line beside the 8 TB/s peak: a plain device-to-device
    copy of the send buffer's size (torch copy_), read + write bytes over its
    median time."""
    n = mib << 20
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    b = torch.empty(n, dtype=torch.uint8, device=dev)
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    times = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        b.copy_(a)
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3)
    us = float(np.median(times))
    del a, b
    return {"gbps": round(2 * n / (us * 1e-6) / 1e9, 1), "us": round(us, 2),
            "pct_of_peak": round(100 * 2 * n / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 2),
            "what": f"torch copy_ of {mib} MiB, read + write bytes, median of {reps}"}


def bench_isolated(ep, torch, hip, ops, names, set_events, dev, stream, reps=30):
    """Each op on its own, its inputs left in place by a previous step, after
    READING a 1 GiB scratch buffer (larger than the 256 MB Infinity Cache plus
    8 x 4 MB of L2), so the op's reads come from HBM.  A read, not a write:
    overwriting the buffer would leave the caches full of dirty lines whose
    write-back the op would then pay for.  Times are the op's own kernels
    (start and stop events recorded by their dispatch packets)."""
    scratch = torch.ones(1 << 28, dtype=torch.int32, device=dev)
    sink = torch.empty((), dtype=torch.int64, device=dev)
    for _ in range(2):
        torch.sum(scratch, dim=0, dtype=torch.int64, out=sink)
    starts = [[hip.create() for _ in ops] for _ in range(reps)]
    stops = [[hip.create() for _ in ops] for _ in range(reps)]
    for r in range(reps):
        for i, op in enumerate(ops):
            torch.sum(scratch, dim=0, dtype=torch.int64, out=sink)
            set_events(starts[r][i], stops[r][i])
            op()
    torch.cuda.synchronize()
    res = {}
    for i, n in enumerate(names):
        v = np.array([hip.elapsed_ms(starts[r][i], stops[r][i]) * 1e3 for r in range(reps)])
        p10, p50, p90 = np.percentile(v, [10, 50, 90])
        res[n] = {"median_us": round(float(p50), 2), "p10_us": round(float(p10), 2),
                  "p90_us": round(float(p90), 2), "p90_over_p10": round(float(p90 / p10), 3)}
    for row in starts + stops:
        for e in row:
            hip.destroy(e)
    del scratch
    res["note"] = (f"{reps} reps per op, each after reading a 1 GiB buffer; the op's own "
                   "kernels from their dispatch packets")
    return res


SYNC_MODES = {0: "item_events", 1: "row_flag", 2: "checksum", 3: "sentinel", 4: "chunk_flag"}


def time_fused(ep, torch, x, idx, wt, E, R, fz, stream, K, W, sync):
    for _ in range(W):
        ep.ep_fused_dispatch_combine(x, idx, wt, E, R, out=fz, stream=stream, sync=sync)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(K):
        ep.ep_fused_dispatch_combine(x, idx, wt, E, R, out=fz, stream=stream, sync=sync)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / K


def bench_fused_workload(ep, torch, w, dev, stream, W, K=10, modes=(0, 1)):
    """The fused mode on a workload of its own (the skewed incast one, 10% of
    the experts taking half of the picks): its own inputs, the library's own
    routing, the same parity gate (combine(dispatch(x)) == x, no device
    error) before timing."""
    from combine_ep_route_topk_amd import workloads as wl
    inp = wl.make_inputs(w)
    logits = torch.from_numpy(inp["logits"]).to(dev)
    x = torch.from_numpy(inp["x"].view(np.int16)).to(dev).view(torch.bfloat16)
    idx, wt = ep.ep_route_topk(logits, w.k, stream=stream)
    res = bench_fused(ep, torch, w, x, idx, wt, stream, K, W, modes)
    res["workload"] = w.describe()
    res["pct_of_peak"] = (round(100 * res["gbps"] / HBM_PEAK_GBPS, 2)
                          if res.get("gbps") else None)
    del x, logits, idx, wt
    torch.cuda.empty_cache()
    return res


def bench_fused(ep, torch, w, x, idx, wt, stream, K, W, modes=tuple(SYNC_MODES)):
    """The fused flag-in-payload mode, the chosen synchronisation variants, on
    the step's inputs (each call after the previous on one stream)."""
    T, H, E, R, k = w.T, w.H, w.E, w.R, w.k
    from combine_ep_route_topk_amd import workloads as wl
    ab = wl.algorithmic_bytes(w)
    byts = ab["layout"] + ab["dispatch"] + ab["combine"] + 16 * w.S
    res = {}
    fz = ep.fused_outputs(T, H, k, E, R, x.device)
    for sync, name in SYNC_MODES.items():
        if sync not in modes:
            continue
        try:
            ep.ep_fused_dispatch_combine(x, idx, wt, E, R, out=fz, stream=stream, sync=sync)
        except ep.EpError as e:
            res[name] = {"status": str(e)}
            continue
        torch.cuda.synchronize()
        if ep.ep_get_device_error(fz["workspace"]) != ep.EP_OK or \
                not torch.equal(fz["out"].view(torch.int16), x.view(torch.int16)):
            res[name] = {"status": "parity gate failed"}
            continue
        us = time_fused(ep, torch, x, idx, wt, E, R, fz, stream, K, W, sync)
        res[name] = {"us_per_call": round(us, 2), "gbps": round(byts / (us * 1e-6) / 1e9, 1)}
    d = res.get("item_events", {})
    return {"us_per_call": d.get("us_per_call"), "gbps": d.get("gbps"),
            "algorithmic_bytes": byts, "traffic": traffic_for("fused", w.name),
            "sync_modes": res,
            "what": "layout + dispatch + combine (identity experts) in one launch"}


def sync_sweep(args):
    """UBEP Fig. 10 on one GPU: latency of layout + dispatch + combine for the
    three-launch path (kernel boundaries as the barriers: stop-and-wait) and
    for the fused mode's synchronisation variants, over the bytes per row
    (H), at the DeepSeek-V3-like T, E, R, k.  Prints one JSON line."""
    import torch

    from combine_ep_route_topk_amd import ep
    from combine_ep_route_topk_amd import workloads as wl
    dev = torch.device("cuda:0")
    base = wl.WORKLOADS[args.workload]
    T, E, R, k = base.T, base.E, base.R, base.k
    stream = torch.cuda.current_stream(dev)
    set_events = ep.library().ep_set_timing_events
    rows = []
    for H in (64, 256, 1024, 2048, 4096, 7168):
        w = wl.Workload(f"{base.name}_H{H}", T=T, H=H, E=E, R=R, k=k, seed=base.seed)
        inp = wl.make_inputs(w)
        x = torch.from_numpy(inp["x"].view(np.int16)).to(dev).view(torch.bfloat16)
        idx, wt = ep.ep_route_topk(torch.from_numpy(inp["logits"]).to(dev), k, True)
        lay = ep.layout_outputs(T, k, E, R, dev)
        send = torch.empty((T * k, H), dtype=torch.bfloat16, device=dev)
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        ops = [ep.bind_dispatch_layout(idx, E, R, lay, stream),
               ep.bind_dispatch(x, lay["pos"], send, stream),
               ep.bind_combine(send, lay["pos"], wt, out, stream)]
        step = make_step(ops, set_events)
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(args.steps):
            step()
        b.record(stream)
        torch.cuda.synchronize()
        row = {"H": H, "row_bytes": 2 * H,
               "stop_and_wait_us": round(a.elapsed_time(b) * 1e3 / args.steps, 2)}
        if not torch.equal(out.view(torch.int16), x.view(torch.int16)):
            row["stop_and_wait_us"] = None
        fz = ep.fused_outputs(T, H, k, E, R, dev)
        for sync, name in SYNC_MODES.items():
            ep.ep_fused_dispatch_combine(x, idx, wt, E, R, out=fz, stream=stream, sync=sync)
            torch.cuda.synchronize()
            ok = ep.ep_get_device_error(fz["workspace"]) == ep.EP_OK and \
                torch.equal(fz["out"].view(torch.int16), x.view(torch.int16))
            row[name + "_us"] = round(time_fused(ep, torch, x, idx, wt, E, R, fz, stream,
                                                 args.steps, args.warmup, sync), 2) if ok else None
        rows.append(row)
        print(f"[sync-sweep] H={H} {row}", file=sys.stderr, flush=True)
        del x, send, out, fz, lay
    print(json.dumps({"sync_sweep": rows, "T": T, "E": E, "R": R, "k": k,
                      "steps": args.steps, "warmup": args.warmup,
                      "what": "layout + dispatch + combine latency (us) per call"}), flush=True)


def partition_sweep(args):
    """UBEP sec. 3.3 / StrataCL sec. 6.2 on one GPU: C persistent "cores"
    copy the send buffer's peer windows (ep_window_copy) following (a) one core
    per peer window, (b) equal slot slices from the GPU search
    (ep_expert_slices), (c) StrataCL's LPT task lists (ep_lpt_partition);
    reports the copy time and the per-core completion-time gap
    (slowest - fastest) / slowest.  Prints one JSON line."""
    import torch

    from combine_ep_route_topk_amd import ep
    from combine_ep_route_topk_amd import workloads as wl
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    hip = ep.HipEvents()
    set_events = ep.library().ep_set_timing_events
    res = []
    for name in ("dsv3", "glm45air", "incast"):
        w = wl.WORKLOADS[name]
        inp = wl.make_inputs(w, with_x=False)
        # the library's own route and layout give the windows
        idx, _ = ep.ep_route_topk(torch.from_numpy(inp["logits"]).to(dev), w.k)
        lay_dev = ep.ep_dispatch_layout(idx, w.E, w.R)
        if ep.ep_get_device_error(lay_dev["workspace"]) != ep.EP_OK:
            raise RuntimeError("layout reported a device error")
        row_bytes = 2 * w.H
        src = torch.randint(-30000, 30000, (w.S, w.H), dtype=torch.int16, device=dev)
        dst = torch.empty_like(src)
        ro = lay_dev["rank_offsets"].cpu().numpy()
        eo_dev = lay_dev["expert_offsets"]
        clock = torch.zeros(2 * 4096, dtype=torch.int64, device=dev)
        bad = torch.zeros(1, dtype=torch.int32, device=dev)

        def timed(C, **kw):
            def call():
                ep.ep_window_copy(src, dst, row_bytes, w.S, C, core_clock=clock[:2 * C], bad=bad,
                                  stream=stream, **kw)
            for _ in range(args.warmup):
                call()
            st, sp = hip.create(), hip.create()
            times = []
            for _ in range(args.steps):
                set_events(st, sp)
                call()
                torch.cuda.synchronize()
                times.append(hip.elapsed_ms(st, sp) * 1e3)
            hip.destroy(st)
            hip.destroy(sp)
            ok = int(bad.item()) == 0 and torch.equal(dst, src)
            c = clock[:2 * C].cpu().numpy().astype(np.float64)
            t0 = c[0::2].min()
            ends = c[1::2] - t0
            gap = float((ends.max() - ends.min()) / ends.max()) if ends.max() > 0 else 0.0
            return {"us": round(float(np.median(times)), 2), "core_gap": round(gap, 3),
                    "gbps": round(2 * w.S * row_bytes / (np.median(times) * 1e-6) / 1e9, 1),
                    "parity": ok}

        row = {"workload": w.describe(), "rank_rows_min_max": [int(np.diff(ro).min()),
                                                               int(np.diff(ro).max())]}
        # (a) one core per peer window
        tasks = np.zeros(w.R, ep.TASK_DTYPE)
        tasks["peer"] = np.arange(w.R)
        tasks["first_row"] = ro[:-1]
        tasks["rows"] = np.diff(ro)
        row["per_peer_C=R"] = timed(w.R, tasks=ep.tasks_to_device(tasks, dev),
                                    core_begin=torch.arange(w.R + 1, dtype=torch.int64, device=dev))
        for C in (w.R, 256):
            # (b) equal slices: the search itself, then the copy
            sl = ep.ep_expert_slices(eo_dev, C, stream=stream)
            st, sp = hip.create(), hip.create()
            set_events(st, sp)
            ep.ep_expert_slices(eo_dev, C, out=sl, stream=stream)
            torch.cuda.synchronize()
            search_us = hip.elapsed_ms(st, sp) * 1e3
            hip.destroy(st)
            hip.destroy(sp)
            r = timed(C, slice_start=sl["start"])
            r["search_us"] = round(search_us, 2)
            row[f"slices_C={C}"] = r
            # (c) LPT task lists, units of 64 rows, cap C/8 units per peer and stripe
            t0 = time.perf_counter()
            tasks, core_begin, _ = ep.ep_lpt_partition(ro, row_bytes, 64, C, alpha=[2000.0],
                                                       beta=[100.0], cap=[max(1, C // 8)])
            host_us = (time.perf_counter() - t0) * 1e6
            r = timed(C, tasks=ep.tasks_to_device(tasks, dev),
                      core_begin=torch.from_numpy(core_begin).to(dev))
            r["schedule_host_us"] = round(host_us, 1)
            r["units"] = int(len(tasks))
            row[f"lpt_C={C}"] = r
            # (d) the same without a binding fan-out cap (C units of a peer per stripe)
            tasks, core_begin, _ = ep.ep_lpt_partition(ro, row_bytes, 64, C, alpha=[2000.0],
                                                       beta=[100.0], cap=[C])
            row[f"lpt_nocap_C={C}"] = timed(C, tasks=ep.tasks_to_device(tasks, dev),
                                            core_begin=torch.from_numpy(core_begin).to(dev))
        res.append(row)
        print(f"[partition] {json.dumps(row)}", file=sys.stderr, flush=True)
        del src, dst
    print(json.dumps({"partition_sweep": res, "steps": args.steps, "warmup": args.warmup,
                      "what": "ep_window_copy of the send buffer (read + write S rows) per schedule"}),
          flush=True)


def cpu_baseline(w, inp, gpu_lay, seconds, step_bytes):
    """The CPU oracle (single-threaded C, double precision) on this host:
    whole steps of the same workload, repeated for about `seconds`."""
    import oracle

    reps, t_total = 0, 0.0
    idx = wt = lay = None
    stage_s = {"route": [], "layout": [], "dispatch": [], "combine": []}
    while reps < 1 or (t_total < seconds and reps < 20):
        t0 = time.perf_counter()
        idx, wt = oracle.route_topk(inp["logits"], w.k, 1)
        t1 = time.perf_counter()
        lay = oracle.dispatch_layout(idx, w.E, w.R)
        t2 = time.perf_counter()
        send = oracle.dispatch(inp["x"], lay["pos"])
        t3 = time.perf_counter()
        oracle.combine(send, lay["pos"], wt)
        t4 = time.perf_counter()
        for name, a, b in (("route", t0, t1), ("layout", t1, t2), ("dispatch", t2, t3),
                           ("combine", t3, t4)):
            stage_s[name].append(b - a)
        t_total += t4 - t0
        reps += 1
    sec_per_step = t_total / reps
    agree = bool(np.array_equal(gpu_lay["pos"].cpu().numpy(), lay["pos"]))
    return {"value": round(step_bytes / sec_per_step / 1e9, 3), "unit": "GB/s",
            "cores": 1, "kind": "oracle",
            "sample": f"{reps} whole steps of {w.name} (route, layout, dispatch, combine), "
                      f"{sec_per_step:.3f} s per step, single thread; host has "
                      f"{os.cpu_count()} cores ({cpu_model()})",
            "stage_median_ms": {n: round(1e3 * float(np.median(v)), 2) for n, v in stage_s.items()},
            "gpu_pos_matches_oracle": agree}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of the MoE routing path on one MI355X: route -> dispatch -> combine.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one pass of the whole path over one batch of synthetic input:
routing (x @ gate_w -> top-K -> renormalised weights), dispatch (counting
sort + row scatter into expert-contiguous order) and combine (weighted
un-permute of the expert outputs y), made as moe_route_dispatch +
moe_combine; the same path as three calls (moe_route, moe_dispatch,
moe_combine) is timed beside it.  The default workload is
N=16384 tokens (8 sequences x 2048), H=4096, E=64, K=2, bf16.  Inputs are
resident in HBM before the timed region; three input sets are rotated so the
256 MiB Infinity Cache never serves a step the data of the previous step.

Prints ONE JSON line: routed tokens/s (value), per-stage times and
algorithmic bandwidth, a roofline object for the dominant kernel (timed with
HIP events on the stream it runs on) and the CPU oracle's throughput on a
bounded sample of the same workload, timed on this host (cpu_baseline).
"""
import argparse
import math
import ctypes
import hashlib
import json
import os
import platform
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA, TFLOP/s
N_SETS = 3
EP_RANKS = 8                  # expert-parallel ranks simulated by moe_ep_dispatch


def algorithmic_bytes(N, H, E, K, b):
    """Bytes each stage must move (logits never leave the chip; each token
    row is read once by dispatch)."""
    T = N * K
    route = N * H * b + H * E * b + T * 8 + E * 4 + E * 4
    dispatch = N * H * b + T * H * b + 3 * T * 4 + (2 * E + 1) * 4
    combine = T * H * b + T * 8 + N * H * b
    return {"route": route, "dispatch": dispatch, "combine": combine}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def traffic_record(kernel, workload):
    """HBM bytes per launch measured with rocprofv3 counters, from the
    committed summary under profiles/, or None if the kernel source changed
    since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.md")
    if not os.path.exists(path):
        return None
    src = os.path.join(ROOT, "moe_token_routing_router_amd", "csrc", f"{kernel}.hip")
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16] if os.path.exists(src) else ""
    for line in open(path):
        m = re.match(r"\|\s*(\w+)\s*\|\s*([\w\-]+)\s*\|\s*([0-9a-f]+)\s*\|\s*([0-9.]+)\s*\|", line)
        if m and m.group(1) == kernel and m.group(2) == workload and m.group(3) == sha:
            return float(m.group(4))
    return None


def cpu_threads():
    """Host threads for the oracle's all-cores run: the cores this process
    may run on, capped by OMP_NUM_THREADS when the host sets it (the share
    of the host that goes with one GPU)."""
    n = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def cpu_baseline(d, min_seconds, threads):
    """The oracle as it stands (plain C, fp64) on the whole workload, repeated
    until at least `min_seconds` have passed.  `threads` > 1 splits the
    router's and the combine's token loops over that many OpenMP threads;
    the counting sort and the row permutation stay sequential."""
    from oracle import oracle as O
    O.set_threads(threads)
    try:
        t0 = time.perf_counter()
        passes = 0
        while True:
            ids, w, _, _ = O.route(d["x"], d["gate_w"], d["bias"], d["K"], d["dtype"])
            _, _, perm, inv = O.dispatch(ids, d["E"])
            O.permute_rows(d["x"], perm, d["K"])
            O.combine(d["y"], inv, w, d["dtype"])
            passes += 1
            el = time.perf_counter() - t0
            if el >= min_seconds:
                break
    finally:
        O.set_threads(1)
    what = "1 thread" if threads == 1 else f"{threads} threads (OpenMP over tokens in route " \
                                            "and combine; counting sort and row copy sequential)"
    return {"value": round(passes * d["N"] / el, 1), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"full workload (N={d['N']}) route+dispatch+combine x {passes} passes, "
                      f"{el:.1f} s on {what} of {cpu_model()}"}


def small_step_graph(L, I, name, steps, dev):
    """One fused forward step (moe_route_dispatch + moe_combine) of a small
    workload: launched call by call through the C ABI, then captured once in
    a HIP graph and replayed.  Returns wall-clock steps/s of both."""
    import torch
    wl = I.WORKLOADS[name]
    d = I.make_inputs(wl)
    N, H, E, K = wl.N, wl.H, wl.E, wl.K
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32

    def to_dev(a):
        if wl.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    x, y, gw = to_dev(d["x"]), to_dev(d["y"]), to_dev(d["gate_w"])
    bias = None if d["bias"] is None else torch.from_numpy(d["bias"]).to(dev)
    i32 = dict(dtype=torch.int32, device=dev)
    ids, w = torch.empty((N, K), **i32), torch.empty((N, K), dtype=torch.float32, device=dev)
    counts, offsets = torch.empty((E,), **i32), torch.empty((E + 1,), **i32)
    perm, inv = torch.empty((N * K,), **i32), torch.empty((N * K,), **i32)
    x_perm = torch.empty((N * K, H), dtype=tdt, device=dev)
    out = torch.empty((N, H), dtype=tdt, device=dev)
    ws = torch.empty((L.moe_route_dispatch_workspace_size(N, H, E, K, tdt),), dtype=torch.uint8,
                     device=dev)
    L.moe_route_dispatch(x, gw, bias, K, ids, w, counts, offsets, perm, inv, x_perm, ws)
    L.moe_combine(y, inv, w, out)
    torch.cuda.synchronize()
    lib = L.library()
    P = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None
    dt = L.MOE_BF16 if wl.dtype == "bf16" else L.MOE_F32

    def args_on(stream_ptr):
        sp = ctypes.c_void_p(stream_ptr)
        return ((P(x), P(gw), P(bias), N, H, E, K, dt, P(ids), P(w), P(counts), P(offsets),
                 P(perm), P(inv), P(x_perm), P(ws), ws.numel(), sp),
                (P(y), P(inv), P(w), N, H, K, dt, P(out), sp))

    def launch(a):
        if lib.moe_route_dispatch(*a[0]) or lib.moe_combine(*a[1]):
            raise RuntimeError("small-workload step failed")

    eager = args_on(torch.cuda.current_stream(dev).cuda_stream)
    for _ in range(10):
        launch(eager)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        launch(eager)
    torch.cuda.synchronize()
    t_eager = time.perf_counter() - t0
    ref = out.clone()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        launch(args_on(torch.cuda.current_stream(dev).cuda_stream))
    for _ in range(10):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    t_graph = time.perf_counter() - t0
    assert torch.equal(out.view(torch.uint8), ref.view(torch.uint8)), "graph replay differs"
    return {"workload": wl.describe(), "eager_steps_per_s": round(steps / t_eager, 1),
            "graph_steps_per_s": round(steps / t_graph, 1),
            "eager_us_per_step": round(t_eager / steps * 1e6, 2),
            "graph_us_per_step": round(t_graph / steps * 1e6, 2)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from moe_token_routing_router_amd import _lib as L
    from moe_token_routing_router_amd import inputs as I

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    lib = L.library()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    wl = I.WORKLOADS[args.workload or I.HEADLINE]
    N, H, E, K = wl.N, wl.H, wl.E, wl.K
    T = N * K
    b = wl.elem_bytes
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    d = I.make_inputs(wl)

    def to_dev(a):
        if wl.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    x0 = to_dev(d["x"])
    y0 = to_dev(d["y"])
    gw = to_dev(d["gate_w"])
    bias = None if d["bias"] is None else torch.from_numpy(d["bias"]).to(dev)

    # N_SETS resident input sets (x, y differ; set 0 is the generated data,
    # the others are row-rotations of it so every set has the same statistics)
    sets = []
    for s in range(N_SETS):
        x = x0 if s == 0 else torch.roll(x0, shifts=997 * s, dims=0).contiguous()
        y = y0 if s == 0 else torch.roll(y0, shifts=991 * s, dims=0).contiguous()
        st = dict(x=x, y=y,
                  ids=torch.empty((N, K), dtype=torch.int32, device=dev),
                  w=torch.empty((N, K), dtype=torch.float32, device=dev),
                  counts=torch.empty((E,), dtype=torch.int32, device=dev),
                  offsets=torch.empty((E + 1,), dtype=torch.int32, device=dev),
                  perm=torch.empty((T,), dtype=torch.int32, device=dev),
                  inv=torch.empty((T,), dtype=torch.int32, device=dev),
                  x_perm=torch.empty((T, H), dtype=tdt, device=dev),
                  out=torch.empty((N, H), dtype=tdt, device=dev))
        sets.append(st)
    rws = torch.empty((max(1, L.moe_route_workspace_size(H, E, tdt)),), dtype=torch.uint8,
                      device=dev)
    dws = torch.empty((L.moe_dispatch_workspace_size(N, E, K),), dtype=torch.uint8, device=dev)
    fws = torch.empty((L.moe_route_dispatch_workspace_size(N, H, E, K, tdt),), dtype=torch.uint8,
                      device=dev)

    # validate every buffer once through the checked binding
    for st in sets:
        L.moe_route(st["x"], gw, bias, K, st["ids"], st["w"], None, rws)
        L.moe_dispatch(st["ids"], st["x"], E, st["counts"], st["offsets"], st["perm"],
                       st["inv"], st["x_perm"], dws)
        L.moe_route_dispatch(st["x"], gw, bias, K, st["ids"], st["w"], st["counts"],
                             st["offsets"], st["perm"], st["inv"], st["x_perm"], fws)
        L.moe_combine(st["y"], st["inv"], st["w"], st["out"])
    torch.cuda.synchronize()

    # then call the C ABI directly with the pointers (no per-call Python checks)
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None
    dt = L.MOE_BF16 if wl.dtype == "bf16" else L.MOE_F32
    calls = []
    for st in sets:
        calls.append(dict(
            route=(P(st["x"]), P(gw), P(bias), N, H, E, K, dt, P(st["ids"]), P(st["w"]), None,
                   P(rws), rws.numel(), sp),
            dispatch=(P(st["ids"]), P(st["x"]), N, H, E, K, dt, P(st["counts"]),
                      P(st["offsets"]), P(st["perm"]), P(st["inv"]), P(st["x_perm"]), P(dws),
                      dws.numel(), sp),
            route_dispatch=(P(st["x"]), P(gw), P(bias), N, H, E, K, dt, P(st["ids"]),
                            P(st["w"]), P(st["counts"]), P(st["offsets"]), P(st["perm"]),
                            P(st["inv"]), P(st["x_perm"]), P(fws), fws.numel(), sp),
            combine=(P(st["y"]), P(st["inv"]), P(st["w"]), N, H, K, dt, P(st["out"]), sp)))
    fn = {"route": lib.moe_route, "dispatch": lib.moe_dispatch,
          "route_dispatch": lib.moe_route_dispatch, "combine": lib.moe_combine}

    def call(name, i):
        status = fn[name](*calls[i % N_SETS][name])
        if status:
            raise RuntimeError(f"{name} returned status {status}")

    def step(i):  # the whole path: fused route+dispatch, then combine
        call("route_dispatch", i)
        call("combine", i)

    def step_unfused(i):  # the same path as three separate calls
        call("route", i)
        call("dispatch", i)
        call("combine", i)

    stream2 = torch.cuda.Stream(dev)  # default priority, like the launch stream
    sp2 = ctypes.c_void_p(stream2.cuda_stream)
    combine2 = [c["combine"][:-1] + (sp2,) for c in calls]
    ev_rd = [torch.cuda.Event() for _ in range(N_SETS)]
    ev_cb = [torch.cuda.Event() for _ in range(N_SETS)]

    def overlapped_steps(n):
        a = torch.cuda.Event(enable_timing=True)
        z = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        a.record(stream)
        for i in range(n):
            j = i % N_SETS
            if i >= N_SETS:
                stream.wait_event(ev_cb[j])  # combine of batch i - N_SETS has read set j
            call("route_dispatch", i)
            ev_rd[j].record(stream)
            stream2.wait_event(ev_rd[j])
            status = lib.moe_combine(*combine2[j])
            if status:
                raise RuntimeError(f"combine returned status {status}")
            ev_cb[j].record(stream2)
        stream.wait_stream(stream2)
        z.record(stream)
        torch.cuda.synchronize()
        return time.perf_counter() - t0, a.elapsed_time(z)

    def timed(fn_step, n):
        a = torch.cuda.Event(enable_timing=True)
        z = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        a.record(stream)
        for i in range(n):
            fn_step(i)
        z.record(stream)
        torch.cuda.synchronize()
        return time.perf_counter() - t0, a.elapsed_time(z)

    for i in range(args.warmup):
        step(i)
        step_unfused(i)
    torch.cuda.synchronize()

    # timed region 1: the whole path, K steps, nothing between the launches
    wall, gpu_ms = timed(step, args.steps)
    # timed region 2: the same path as three separate calls
    wall_u, gpu_ms_u = timed(step_unfused, args.steps)
    # context (not the headline): consecutive batches overlapped as a caller
    # pipelining its steps would run them -- moe_route_dispatch of batch i+1 on
    # the launch stream while moe_combine of batch i runs on a second stream
    # (default priority), with events for the data each needs and for the
    # reuse of a set's buffers three batches later
    overlapped_steps(2 * N_SETS)  # untimed warm-up of the two-stream schedule
    wall_o, gpu_ms_o = overlapped_steps(args.steps)
    # timed region 3: each call on its own, K back-to-back calls (rotating the
    # input sets) between one pair of HIP events on the launch stream: the
    # average duration of one call
    stage_ms = {}
    for name in ("route_dispatch", "combine", "route", "dispatch"):
        for i in range(3):
            call(name, i)
        _, ms = timed(lambda i, n=name: call(n, i), args.steps)
        stage_ms[name] = ms / args.steps
    # the spread of single calls: one pair of HIP events around each call
    # (the events add a little to every call, so the back-to-back average
    # above is the figure of record)
    stage_dist = {}
    for name in ("route_dispatch", "combine", "route", "dispatch"):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i, (a, z) in enumerate(evs):
            a.record(stream)
            call(name, i)
            z.record(stream)
        torch.cuda.synchronize()
        us = np.array([a.elapsed_time(z) * 1e3 for a, z in evs])
        stage_dist[name] = {"p10_us": round(float(np.percentile(us, 10)), 2),
                            "p50_us": round(float(np.percentile(us, 50)), 2),
                            "p90_us": round(float(np.percentile(us, 90)), 2)}

    # Cache-cold single calls: before each call an untimed read of 1 GiB (four
    # times the 256 MiB Infinity Cache, the memory-side cache in front of
    # HBM) evicts what earlier calls left there, so every input a call reads
    # comes from HBM.  A read, not a write: a written scrub would leave the
    # cache full of dirty lines whose write-back the timed call would pay.
    # One HIP event pair around each call, median reported.
    # "dispatch_after_route" runs moe_route untimed between the scrub and the
    # timed moe_dispatch, so the scatter's read of x follows the router's
    # read of the same 128 MiB -- the warm case of the unfused pipeline.
    scrub = torch.zeros((1 << 28,), dtype=torch.float32, device=dev)
    scrub_out = torch.empty((), dtype=torch.float32, device=dev)
    for _ in range(3):  # write back the zero fill before any timing
        torch.sum(scrub, dim=0, out=scrub_out)

    def cold_us(name, n, before=None):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        torch.cuda.synchronize()
        for i, (a, z) in enumerate(evs):
            torch.sum(scrub, dim=0, out=scrub_out)
            if before is not None:
                call(before, i)
            a.record(stream)
            call(name, i)
            z.record(stream)
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(z) * 1e3 for a, z in evs]))

    cold = {name: cold_us(name, args.steps) for name in ("route_dispatch", "route", "dispatch",
                                                         "combine")}
    cold["dispatch_after_route"] = cold_us("dispatch", args.steps, before="route")
    del scrub, scrub_out

    # The other calls of the library, each measured on its own.  Their
    # buffers are allocated only now, so the timed regions above run with the
    # same memory layout whether or not these exist.
    # expert-parallel send metadata (measured on its own, not part of the step)
    R = EP_RANKS if E % EP_RANKS == 0 else 1
    cap = N * min(K, R)
    for st in sets:
        st.update(send_counts=torch.empty((R,), dtype=torch.int32, device=dev),
                  send_offsets=torch.empty((R + 1,), dtype=torch.int32, device=dev),
                  send_tok=torch.empty((cap,), dtype=torch.int32, device=dev),
                  send_row=torch.empty((T,), dtype=torch.int32, device=dev),
                  expand_idx=torch.empty((T,), dtype=torch.int32, device=dev),
                  x_send=torch.empty((cap, H), dtype=tdt, device=dev))
    ews = torch.empty((L.moe_ep_dispatch_workspace_size(N, E, K, R),), dtype=torch.uint8,
                      device=dev)
    # backward of the path (measured on its own): upstream gradients are the
    # other sets' rows (dout = a token matrix, dx_perm = a dispatched matrix)
    for s_i, st in enumerate(sets):
        other = sets[(s_i + 1) % N_SETS] if N_SETS > 1 else st
        st.update(dout=other["x"], dx_perm=other["y"],
                  dtopk_w=torch.randn((N, K), dtype=torch.float32, device=dev),
                  dy=torch.empty((T, H), dtype=tdt, device=dev),
                  dw=torch.empty((N, K), dtype=torch.float32, device=dev),
                  dx=torch.empty((N, H), dtype=tdt, device=dev),
                  dgate=torch.empty((H, E), dtype=torch.float32, device=dev),
                  dbias=torch.empty((E,), dtype=torch.float32, device=dev))
    bws = torch.empty((L.moe_route_backward_workspace_size(N, H, E, K, tdt),), dtype=torch.uint8,
                      device=dev)
    # the expert layer between dispatch and combine (measured on its own):
    # one linear map per expert, F = H outputs, synthetic N(0, 1/H) weights
    # drawn on the device from a seeded generator (no checkpoint)
    F = H
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    wexp = (torch.randn((E, F, H), generator=gen, device=dev, dtype=torch.float32)
            / math.sqrt(H)).to(tdt)
    for st in sets:
        st.update(yexp=torch.empty((T, F), dtype=tdt, device=dev),
                  agg=torch.empty((N, H), dtype=tdt, device=dev))
    for st in sets:
        L.moe_ep_dispatch(st["ids"], st["x"], E, R, st["counts"], st["offsets"], st["perm"],
                          st["inv"], st["send_counts"], st["send_offsets"], st["send_tok"],
                          st["send_row"], st["expand_idx"], st["x_send"], ews)
        L.moe_grouped_linear(st["x_perm"], wexp, st["offsets"], st["yexp"])
        L.moe_aggregate(st["y"], st["inv"], st["w"], st["x"], st["agg"])
        L.moe_combine_backward(st["dout"], st["y"], st["inv"], st["w"], st["dy"], st["dw"])
        L.moe_dispatch_backward(st["dx_perm"], st["inv"], st["dx"])
        L.moe_route_backward(st["x_perm"], gw, st["ids"], st["w"], st["dtopk_w"], st["perm"],
                             st["offsets"], st["inv"], st["dx_perm"], st["dgate"], st["dbias"],
                             st["dx"], bws)
    torch.cuda.synchronize()
    for c, st in zip(calls, sets):
        c.update(
            ep_dispatch=(P(st["ids"]), P(st["x"]), N, H, E, K, R, dt, P(st["counts"]),
                         P(st["offsets"]), P(st["perm"]), P(st["inv"]), P(st["send_counts"]),
                         P(st["send_offsets"]), P(st["send_tok"]), P(st["send_row"]),
                         P(st["expand_idx"]), P(st["x_send"]), P(ews), ews.numel(), sp),
            grouped_linear=(P(st["x_perm"]), P(wexp), P(st["offsets"]), T, H, E, F, dt,
                            P(st["yexp"]), sp),
            aggregate=(P(st["y"]), P(st["inv"]), P(st["w"]), P(st["x"]), N, H, K, dt,
                       P(st["agg"]), sp),
            combine_backward=(P(st["dout"]), P(st["y"]), P(st["inv"]), P(st["w"]), N, H, K, dt,
                              P(st["dy"]), P(st["dw"]), sp),
            dispatch_backward=(P(st["dx_perm"]), P(st["inv"]), N, H, K, dt, P(st["dx"]), sp),
            route_backward=(P(st["x_perm"]), P(gw), P(st["ids"]), P(st["w"]), P(st["dtopk_w"]),
                            P(st["perm"]), P(st["offsets"]), P(st["inv"]), P(st["dx_perm"]), N,
                            H, E, K, dt, P(st["dgate"]), P(st["dbias"]), P(st["dx"]), P(bws),
                            bws.numel(), sp))
    fn.update(ep_dispatch=lib.moe_ep_dispatch, combine_backward=lib.moe_combine_backward,
              grouped_linear=lib.moe_grouped_linear, aggregate=lib.moe_aggregate,
              dispatch_backward=lib.moe_dispatch_backward, route_backward=lib.moe_route_backward)
    for name in ("ep_dispatch", "combine_backward", "dispatch_backward", "route_backward",
                 "aggregate", "grouped_linear"):
        for i in range(3):
            call(name, i)
        _, ms = timed(lambda i, n=name: call(n, i), args.steps)
        stage_ms[name] = ms / args.steps
    # the router with its gate packed once beforehand (moe_route_pack_gate:
    # inference, or a training step that packs the gate right after the
    # weight update): context, not part of the step; only where moe_route
    # packs the gate on every call
    if L.moe_route_workspace_size(H, E, tdt):
        packed = L.pack_gate(gw)
        torch.cuda.synchronize()
        for c, st in zip(calls, sets):
            c.update(
                route_prepacked=(P(st["x"]), P(packed), packed.numel(), P(bias), N, H, E, K, dt,
                                 P(st["ids"]), P(st["w"]), None, sp),
                route_dispatch_prepacked=(P(st["x"]), P(packed), packed.numel(), P(bias), N, H,
                                          E, K, dt, P(st["ids"]), P(st["w"]), P(st["counts"]),
                                          P(st["offsets"]), P(st["perm"]), P(st["inv"]),
                                          P(st["x_perm"]), P(fws), fws.numel(), sp))
        fn.update(route_prepacked=lib.moe_route_prepacked,
                  route_dispatch_prepacked=lib.moe_route_dispatch_prepacked)
        for name in ("route_prepacked", "route_dispatch_prepacked"):
            for i in range(3):
                call(name, i)
            _, ms = timed(lambda i, n=name: call(n, i), args.steps)
            stage_ms[name] = ms / args.steps
    # context for the grouped GEMM: the platform library's dense GEMM of the
    # same total shape (all T rows through one expert's F x H weights), i.e.
    # what a tuned library GEMM reaches without per-expert segments
    dense_ms = None
    if tdt == torch.bfloat16:
        w0 = wexp[0]
        dense = lambda i: torch.mm(sets[i % N_SETS]["x_perm"], w0.t(), out=sets[i % N_SETS]["yexp"])
        for i in range(3):
            dense(i)
        _, ms = timed(dense, args.steps)
        dense_ms = ms / args.steps
    # leave every set's outputs consistent for the check below
    for i in range(N_SETS):
        step(i)
    torch.cuda.synchronize()
    # the small workloads are launch-bound: one step launched call by call
    # against the same step replayed from a HIP graph
    graphs = {n: small_step_graph(L, I, n, max(args.steps, 200), dev)
              for n in ("tiny-fp32", "small-bf16")}

    # correctness guard on the outputs (cheap invariants only)
    last = sets[0]
    cnt = last["counts"].cpu().numpy()
    assert cnt.sum() == T, "token conservation violated"
    load = cnt.astype(np.float64)

    alg = algorithmic_bytes(N, H, E, K, b)
    alg["route_dispatch"] = alg["route"] + alg["dispatch"]
    alg["route_prepacked"] = alg["route"]
    alg["route_dispatch_prepacked"] = alg["route_dispatch"]
    # ep_dispatch: ids in, x read once, S deduplicated rows out, the expert
    # metadata (counts, offsets, perm, inv) and the send metadata (send
    # counts/offsets, send_tok [S], send_row and expand_idx [N*K])
    alg["aggregate"] = alg["combine"] + N * H * b
    alg["grouped_linear"] = T * H * b + E * F * H * b + T * F * b + (E + 1) * 4
    # backward: what each call must move (its scratch excluded)
    alg["combine_backward"] = N * H * b + 2 * T * H * b + 3 * T * 4
    alg["dispatch_backward"] = T * H * b + N * H * b + T * 4
    alg["route_backward"] = (2 * T * H * b + N * H * b + H * E * b + 5 * T * 4 + (E + 1) * 4
                             + H * E * 4 + E * 4)
    S = int(sets[0]["send_offsets"][R].item())
    alg["ep_dispatch"] = (T * 4 + N * H * b + S * H * b + (2 * E + 1) * 4 + 2 * T * 4
                          + (2 * R + 1) * 4 + S * 4 + 2 * T * 4)
    stages = {}
    for k, ms in stage_ms.items():
        stages[k] = {"ms_per_call": round(ms, 5), "alg_MB": round(alg[k] / 1e6, 3),
                     "alg_GBs": round(alg[k] / ms / 1e6, 1),
                     "hbm_frac": round(alg[k] / ms / 1e6 / HBM_PEAK_GBS, 4)}
    # what dispatch adds to the fused call: moe_route_dispatch minus moe_route
    # (the router's epilogue does the ranking, so the count launch disappears).
    # Cache-warm by construction: the scatter re-reads x right after the
    # router read it, and the Infinity Cache (256 MiB) can serve that re-read,
    # so this is an algorithmic rate, not an HBM fraction.
    if "route_dispatch" in stage_ms and "route" in stage_ms:
        marg = stage_ms["route_dispatch"] - stage_ms["route"]
        stages["dispatch_marginal_in_fused_call"] = {
            "ms_per_call": round(marg, 5), "alg_MB": round(alg["dispatch"] / 1e6, 3),
            "alg_GBs": round(alg["dispatch"] / marg / 1e6, 1),
            "alg_frac_of_hbm_peak": round(alg["dispatch"] / marg / 1e6 / HBM_PEAK_GBS, 4),
            "cache_warm": True,
            "note": "x re-read right after the router's read of it; may be served by the "
                    "Infinity Cache, so not an HBM fraction"}
    stages_cold = {}
    for k, us in cold.items():
        a_k = alg["dispatch" if k == "dispatch_after_route" else k]
        stages_cold[k] = {"p50_us": round(us, 2), "alg_GBs": round(a_k / us / 1e3, 1),
                          "hbm_frac": round(a_k / us / 1e3 / HBM_PEAK_GBS, 4)}
    stages_cold["dispatch_after_route"].update(
        cache_warm=True, note="moe_route ran between the scrub and this call: the scatter's "
                              "read of x follows the router's; not an HBM fraction")
    stages_cold["dispatch_after_route"]["alg_frac_of_hbm_peak"] = \
        stages_cold["dispatch_after_route"].pop("hbm_frac")
    stages_cold["route_dispatch"]["note"] = (
        "cold inputs, but the call's own scatter re-reads x right after its router: that "
        "re-read is cache-warm")
    # the fused calls' bytes follow the per-stage model (route + dispatch, x
    # counted by both); their second read of x is served largely by the
    # Infinity Cache, so the fraction is not all HBM traffic
    for k in ("route_dispatch", "route_dispatch_prepacked"):
        if k in stages:
            stages[k].update(cache_warm=True, note=(
                "bytes of route + dispatch (x counted by both); the call's scatter re-reads "
                "x right after its router, largely from the Infinity Cache: not all HBM"))
    stages["ep_dispatch"].update(ep_size=R, send_rows=S, slots=T)
    for k in ("route_prepacked", "route_dispatch_prepacked"):
        if k in stages:
            packed_note = ("gate packed once before the timed calls (moe_route_pack_gate); "
                           "context, not part of the step")
            stages[k]["note"] = (packed_note + "; " + stages[k]["note"]
                                 if "note" in stages[k] else packed_note)
    g_flops = 2.0 * T * H * F
    stages["grouped_linear"].update(
        F=F, tflops=round(g_flops / (stage_ms["grouped_linear"] * 1e-3) / 1e12, 1),
        mfma_frac=round(g_flops / (stage_ms["grouped_linear"] * 1e-3)
                        / (BF16_MFMA_PEAK_TFLOPS * 1e12), 4))
    if dense_ms is not None:
        stages["grouped_linear"]["dense_library_gemm_tflops"] = round(
            g_flops / (dense_ms * 1e-3) / 1e12, 1)
    r_flops = 2.0 * N * H * E
    stages["route"]["mfma_util"] = round(
        r_flops / (stage_ms["route"] * 1e-3) / (BF16_MFMA_PEAK_TFLOPS * 1e12), 4)

    # dominant kernel: combine (one launch per call, the largest kernel of
    # the path)
    kern = "combine"
    avg_ms = stage_ms[kern]
    achieved = alg[kern] / (avg_ms * 1e-3) / 1e9
    traffic = traffic_record(kern, wl.name)
    roofline = {"kernel": "combine_kernel<bf16>" if wl.dtype == "bf16" else "combine_kernel<f32>",
                "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic, "alg_bytes_per_launch": alg[kern],
                "avg_launch_ms": round(avg_ms, 5)}

    # Context: plain PyTorch kernels with the stages' read:write mixes on
    # buffers of the same size (rotating three sets, like the path): a 1:1
    # copy, dispatch's 1:2 fan-out (index_select repeating each row twice),
    # combine's 2:1 as the sum of row pairs and, for K >= 2, as an elementwise
    # add of two contiguous halves of y (a plain streaming kernel).
    # Algorithmic GB/s.
    def plain_gbs(fn, nbytes, n=20):
        for i in range(3):
            fn(i)
        _, ms = timed(fn, n)
        return round(nbytes / (ms / n * 1e-3) / 1e9, 1)
    rep2 = torch.arange(N, device=dev).repeat_interleave(K)
    ceilings = {
        "copy_1to1": plain_gbs(lambda i: sets[i % N_SETS]["out"].copy_(sets[i % N_SETS]["x"]),
                               2 * N * H * b),
        "fanout_1toK": plain_gbs(
            lambda i: torch.index_select(sets[i % N_SETS]["x"], 0, rep2,
                                         out=sets[i % N_SETS]["x_perm"]), N * H * b + T * H * b),
        "sum_Kto1": plain_gbs(
            lambda i: torch.sum(sets[i % N_SETS]["y"].view(N, K, H), dim=1,
                                out=sets[i % N_SETS]["out"]), T * H * b + N * H * b),
        "note": "plain PyTorch kernels, same sizes, read:write mixes of copy, dispatch, combine",
    }
    if K >= 2:
        ceilings["add_2to1"] = plain_gbs(
            lambda i: torch.add(sets[i % N_SETS]["y"][:N], sets[i % N_SETS]["y"][N:2 * N],
                                out=sets[i % N_SETS]["out"]), 3 * N * H * b)
    # leave the outputs of the path consistent for the check below
    for i in range(N_SETS):
        step(i)
    torch.cuda.synchronize()

    if args.copy_calibration:
        a = torch.empty((256 << 20,), dtype=torch.uint8, device=dev)
        bb = torch.empty_like(a)
        for _ in range(3):
            bb.copy_(a)
        torch.cuda.synchronize()

    ms_per_step = wall * 1e3 / args.steps
    alg_step = alg["route"] + alg["dispatch"] + alg["combine"]
    res = {
        "metric": "routed tokens/s (route+dispatch+combine)",
        "value": round(N * args.steps / wall, 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.dtype, "data": "synthetic (seeded, resident in HBM, 3 rotating sets)",
        "config": {"workload": wl.describe(), "N": N, "H": H, "E": E, "K": K,
                   "bias": wl.bias, "name": wl.name},
        "pipeline": {"calls": "moe_route_dispatch + moe_combine",
                     "gpu_ms_per_step": round(gpu_ms / args.steps, 5),
                     "alg_MB_per_step": round(alg_step / 1e6, 3),
                     "alg_frac_of_hbm_peak": round(alg_step / (gpu_ms / args.steps * 1e-3)
                                                   / 1e9 / HBM_PEAK_GBS, 4),
                     "note": "algorithmic bytes over the step time; the dispatch's re-read "
                             "of x inside moe_route_dispatch is cache-warm (no other input "
                             "of a step was touched by the two steps before it)"},
        "pipeline_unfused": {"calls": "moe_route + moe_dispatch + moe_combine",
                             "ms_per_step": round(wall_u * 1e3 / args.steps, 5),
                             "gpu_ms_per_step": round(gpu_ms_u / args.steps, 5),
                             "tokens_per_s": round(N * args.steps / wall_u, 1)},
        "pipeline_overlapped": {
            "calls": "moe_route_dispatch (batch i+1) overlapped with moe_combine (batch i) on a "
                     "second stream; context, not the headline value",
            "ms_per_step": round(wall_o * 1e3 / args.steps, 5),
            "gpu_ms_per_step": round(gpu_ms_o / args.steps, 5),
            "tokens_per_s": round(N * args.steps / wall_o, 1)},
        "stages": stages,
        "stages_cache_cold": stages_cold,
        "stage_spread_us": stage_dist,
        "plain_kernel_ceilings_GBs": ceilings,
        "load_max_over_mean": round(float(load.max() / load.mean()), 3),
        "small_workloads_graph": graphs,
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if not args.no_cpu:
        nt = cpu_threads()
        res["cpu_baseline"] = cpu_baseline(d, args.cpu_seconds, nt)
        res["cpu_baseline"]["single_thread"] = cpu_baseline(d, args.cpu_seconds, 1)
        res["cpu_baseline"]["cpu_model"] = cpu_model()
        res["cpu_baseline"]["affinity_cores"] = len(os.sched_getaffinity(0))
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

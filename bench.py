#!/usr/bin/env python3
"""Benchmark of the skinny decode projection on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-sweep] [--no-cpu-baseline]

Workload (one "step" = one pass of the hot path over one batch): the
small-batch decode projection y = x W^T at M = 1 and M = 2 with K = 7168,
N = 8192, bf16 x ~ N(0, 1) and W ~ N(0, 0.02^2), fp32 and bf16 outputs --
one call of skinny_gemm per batch size, each planned by skinny_gemm_plan
(the small-matrix kernel).  Weights already sit in HBM when timing starts.
Each call reads the next copy of a ring of byte-identical weight copies
larger than twice the 256 MB Infinity Cache, so every call streams its
weights from HBM rather than from cache.

Timing: W warmup steps, then synchronize and time exactly K steps between
two HIP events recorded on the stream the kernels run on.  A short GPU sleep
queued first lets the host enqueue the whole region ahead, so the kernels run
back to back and the events see GPU time only; no event sits between two
launches (on this GPU an event between kernels adds several microseconds of
gap).  The average launch duration is the region's time over its launches.
value = algorithmic bytes of the K steps / their GPU time (GB/s).

The one JSON line also carries a sweep over the other workloads (batch
M = 1..64, residual, MoE grouped), the roofline of the dominant kernel, and
the CPU oracle timed on a bounded sample on this host.

    python bench.py --summarize-pmc FETCH_DIR WRITE_DIR   # rocprofv3 --pmc CSVs -> traffic
    python bench.py --summarize-trace DIR "COMMAND"       # rocprofv3 kernel stats -> table
    python bench.py --profile-workloads MANIFEST           # workloads for rocprofv3 --pmc
    python bench.py --summarize-workloads MANIFEST DIR...  # per-workload counters -> table
"""
from __future__ import annotations

import argparse
import csv
import ctypes
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published peak
MALL_BYTES = 256 * 2 ** 20     # Infinity Cache
RING_MIN_BYTES = 2 * MALL_BYTES + 1
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "gemv_m1m2_k7168_n8192_traffic.txt")
GEMV_SOURCES = ["skinny_gemm_projection_amd/csrc/rowdot.hip", "skinny_gemm_projection_amd/csrc/sg_device.h"]

M_LIST, N_MAIN, K_MAIN = (1, 2), 8192, 7168


def kernel_source_hash(paths=GEMV_SOURCES) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def proj_bytes(M, N, K, f32=True, bf16=True, residual=False) -> int:
    """Algorithmic bytes of one projection: W once, x once, outputs (and r) once."""
    b = N * K * 2 + M * K * 2
    b += M * N * ((4 if f32 else 0) + (2 if bf16 else 0))
    if residual:
        b += M * N * 2
    return b


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# --------------------------------------------------------------------------- GPU timing


class Launcher:
    """Raw C-ABI calls with pointers resolved up front (keeps host overhead low)."""

    def __init__(self, torch, sg):
        self.torch = torch
        self.sg = sg
        self.c = sg._lib.load()
        self.stream = torch.cuda.current_stream()
        self.sp = self.stream.cuda_stream

    def projection(self, plan, x, W, y32, y16, ws=None):
        c, pp = self.c, ctypes.byref(plan)
        args = (pp, x.data_ptr(), W.data_ptr(), y32.data_ptr() if y32 is not None else None,
                y16.data_ptr() if y16 is not None else None,
                ws.data_ptr() if ws is not None else None,
                ws.numel() if ws is not None else 0, self.sp)

        def go():
            st = c.skinny_gemm(*args)
            if st:
                raise RuntimeError(self.sg.skinny_gemm_status_str(st))
        return go

    def residual(self, plan, x, W, r, o16, o32, ws=None):
        c, pp = self.c, ctypes.byref(plan)
        args = (pp, x.data_ptr(), W.data_ptr(), r.data_ptr(), o16.data_ptr(),
                o32.data_ptr() if o32 is not None else None,
                ws.data_ptr() if ws is not None else None,
                ws.numel() if ws is not None else 0, self.sp)

        def go():
            st = c.skinny_gemm_residual(*args)
            if st:
                raise RuntimeError(self.sg.skinny_gemm_status_str(st))
        return go

    def read_probe(self, W, rows_per_iter, grid):
        c = self.c
        args = (W.data_ptr(), W.shape[0], W.shape[1] * W.element_size(), rows_per_iter, grid,
                self.sp)

        def go():
            st = c.skinny_gemm_read_probe(*args)
            if st:
                raise RuntimeError(self.sg.skinny_gemm_status_str(st))
        return go

    def grouped(self, x, W, ids, out, ws):
        c = self.c
        T, K = x.shape
        E, N, _ = W.shape
        topk = ids.shape[1]
        args = (x.data_ptr(), T, W.data_ptr(), E, N, K, ids.data_ptr(), topk, out.data_ptr(),
                None, None, None, ws.data_ptr(), ws.numel(), self.sp)

        def go():
            st = c.grouped_skinny_gemm(*args)
            if st:
                raise RuntimeError(self.sg.skinny_gemm_status_str(st))
        return go

    def moe_step(self, x, Wr, We, Ws, topk, outs, ws, mode):
        """skinny_moe_step: the shared expert fused into the router GEMM (Wr and Ws
        adjacent, outputs in one [T, E + N_shared] buffer), on the binding's side
        stream, serial after the routed experts, or inside the routed-expert launch
        (shared_in_routed, up to 4 tokens)."""
        c, sg = self.c, self.sg
        T, K = x.shape
        E, N, _ = We.shape
        ids, scores, out, shared = outs
        fused = mode == "fused"
        step = sg.SgMoeStep(x.data_ptr(), Wr.data_ptr(), We.data_ptr(),
                            None if fused else Ws.data_ptr(), scores.data_ptr(), ids.data_ptr(),
                            None, out.data_ptr(), None if fused else shared.data_ptr(),
                            T, K, E, topk, N, Ws.shape[0],
                            sg._lib.SG_MOE_STEP_FUSED_SHARED if fused
                            else sg._lib.SG_MOE_STEP_SHARED_IN_ROUTED
                            if mode == "shared_in_routed" else 0)
        side = fork = join = None
        if mode == "side_stream":
            s_, f_, j_ = sg._side_resources(x.device)
            side, fork, join = s_.cuda_stream, f_.cuda_event, j_.cuda_event
        ref = ctypes.byref(step)

        def go(step=step):
            st = c.skinny_moe_step(ref, ws.data_ptr(), ws.numel(), self.sp, side, fork, join)
            if st:
                raise RuntimeError(sg.skinny_gemm_status_str(st))
        return go


def lowp_plan_label(fmt: str, M: int, N: int, wsb: int) -> str:
    """Kernel an FP8 / MXFP4 call runs, as the library routes it (the chunk kernel for
    FP8 from 8 rows, from 12 where N/32 is a whole multiple of 256, K short enough for
    its LDS; for MXFP4 from 17 rows, 12 when N > 5888, 9 where its matrix-core grid is
    not a whole multiple of 256)."""
    tiles32 = (N + 31) // 32
    tiles = tiles32 if tiles32 >= 256 else (N + 15) // 16
    fp8_from = 12 if tiles32 >= 256 and tiles32 % 256 == 0 else 8
    mx_from = 9 if tiles % 256 else 17
    chunk = M >= 17 or (M >= 12 and N > 5888) or (fmt == "fp8" and M >= fp8_from) or \
        (fmt == "mxfp4" and M >= mx_from)
    if chunk:
        return "lowp_chunk + reduce" if wsb else "lowp_chunk"
    if fmt == "fp8":
        return "fp8_mfma" if M >= 5 else "fp8_rowdot"
    return "mxfp4_mfma" if M >= 9 else "mxfp4_rowdot"


def sleep_cycles_per_ms(torch) -> float:
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    torch.cuda._sleep(2_000_000)
    e.record()
    torch.cuda.synchronize()
    return 2_000_000 / max(s.elapsed_time(e), 1e-3)


def timed_calls(torch, calls, reps, cycles_per_ms, warmup=3):
    """Run calls[i % len(calls)] reps times back to back between one event pair.

    No event sits between two calls (an event between kernels adds a gap of
    several microseconds on this GPU), so the average is the steady-state time
    of one call as the stream sees it.  Returns the average GPU ms per call."""
    for i in range(warmup):
        calls[i % len(calls)]()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int(cycles_per_ms * min(50.0, 0.03 * reps + 0.5)))
    start.record()
    for i in range(reps):
        calls[i % len(calls)]()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / reps


def ring_copies(torch, W, min_bytes=RING_MIN_BYTES):
    nbytes = W.numel() * W.element_size()
    count = max(1, math.ceil(min_bytes / nbytes))
    return [W] + [W.clone() for _ in range(count - 1)]


# --------------------------------------------------------------------------- workloads


def main_workload(torch, sg, si, L, steps, warmup, cyc):
    dev = "cuda"
    x = {M: si.normal_bf16((M, K_MAIN), 1.0, si.seed_for(2, si.TAG_X) + M, dev) for M in M_LIST}
    W0 = si.normal_bf16((N_MAIN, K_MAIN), 0.02, si.seed_for(2, si.TAG_W), dev)
    ring = ring_copies(torch, W0)
    plans = {M: sg.skinny_gemm_plan(M, N_MAIN, K_MAIN) for M in M_LIST}
    y32 = {M: torch.empty((M, N_MAIN), device=dev) for M in M_LIST}
    y16 = {M: torch.empty((M, N_MAIN), device=dev, dtype=torch.bfloat16) for M in M_LIST}
    # one launch closure per (batch size, ring copy); step i uses copies 2i, 2i+1 (mod ring)
    R = len(ring)
    calls = {(M, r): L.projection(plans[M], x[M], ring[r], y32[M], y16[M]) for M in M_LIST
             for r in range(R)}
    seq = []
    for i in range(steps):
        for j, M in enumerate(M_LIST):
            seq.append((M, (len(M_LIST) * i + j) % R))

    for i in range(warmup):
        for j, M in enumerate(M_LIST):
            calls[(M, (len(M_LIST) * i + j) % R)]()
    torch.cuda.synchronize()
    sg.skinny_gemm_reset_counters()

    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()                       # barrier (one rank) + synchronize
    t0 = time.perf_counter()
    # a short GPU sleep lets the host queue the whole region before the GPU reaches it, so
    # kernels run back to back and the two events measure GPU time only
    torch.cuda._sleep(int(cyc * min(200.0, 0.02 * len(seq) + 1.0)))
    start.record()
    for key in seq:
        calls[key]()
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(stop)
    counters = sg.skinny_gemm_get_counters()
    assert counters[sg.SG_KERNEL_GEMV] == len(seq), counters
    # per batch size: the same ring, each size alone, for the us/projection breakdown
    per_m_ms = {}
    for M in M_LIST:
        per_m_ms[M] = timed_calls(torch, [calls[(M, r)] for r in range(R)], 200, cyc)
    # the same weight stream with no arithmetic: the read probe on each plan's grid and
    # rows per iteration, over the same ring
    probe_ms = {M: timed_calls(torch, [L.read_probe(ring[r], plans[M].tile_n, plans[M].grid)
                                       for r in range(R)], 200, cyc) for M in M_LIST}
    graph = graph_timing(torch, sg, lambda L2, M, r: L2.projection(plans[M], x[M], ring[r], y32[M],
                                                                    y16[M]),
                         M_LIST, R, y32)

    cold = cold_latency(torch, sg, L, calls, M_LIST, ring)

    bytes_per = {M: proj_bytes(M, N_MAIN, K_MAIN) for M in M_LIST}
    step_bytes = sum(bytes_per.values())
    us = {M: 1e3 * per_m_ms[M] for M in M_LIST}
    launches = len(seq)
    avg_launch_ms = total_ms / launches
    launch_bytes = sum(bytes_per[M] for M, _ in seq) / launches
    achieved = launch_bytes / (avg_launch_ms * 1e-3) / 1e9
    ms_per_step = total_ms / steps
    return {
        "plans": {M: plans[M].as_dict() for M in M_LIST},
        "ring_copies": R, "ring_bytes": R * W0.numel() * 2,
        "ms_per_step": ms_per_step, "wall_ms_per_step": 1e3 * wall / steps,
        "value": step_bytes * steps / (total_ms * 1e-3) / 1e9,
        "us_per_projection": {str(M): round(us[M], 3) for M in M_LIST},
        "gbs_per_batch": {str(M): round(bytes_per[M] / (us[M] * 1e-6) / 1e9, 1) for M in M_LIST},
        "read_probe": {str(M): {"grid": plans[M].grid, "rows_per_iter": plans[M].tile_n,
                                "us": round(1e3 * probe_ms[M], 3),
                                "GBps": round(W0.numel() * 2 / (probe_ms[M] * 1e-3) / 1e9, 1),
                                "projection_over_probe": round(per_m_ms[M] / probe_ms[M], 4)}
                       for M in M_LIST},
        "achieved": achieved, "avg_launch_us": 1e3 * avg_launch_ms,
        "bytes_per_launch": launch_bytes,
        "graph": graph,
        "cold": cold,
        "inputs": (x, W0),
    }


def cold_latency(torch, sg, L, calls, m_list, ring, trials=15):
    """Secondary number: one call on its own, its weights cold.  Before each trial the
    prefetch kernel reads every other copy of the ring (more than the 256 MB Infinity
    Cache), then one event pair brackets the single call (launch latency included).
    Median, min and max us per batch size."""
    R = len(ring)
    nbytes = ring[0].numel() * ring[0].element_size()
    out = {}
    for M in m_list:
        times = []
        for t in range(trials):
            r = t % R
            for o in range(R):
                if o != r:
                    st = L.c.skinny_gemm_prefetch(ring[o].data_ptr(), nbytes, L.sp)
                    if st:
                        raise RuntimeError(sg.skinny_gemm_status_str(st))
            torch.cuda.synchronize()
            start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            start.record()
            calls[(M, r)]()
            stop.record()
            torch.cuda.synchronize()
            times.append(1e3 * start.elapsed_time(stop))
        times.sort()
        out[str(M)] = {"median_us": round(times[len(times) // 2], 3), "min_us": round(times[0], 3),
                       "max_us": round(times[-1], 3)}
    return out


def graph_timing(torch, sg, make_call, m_list, R, y32, per_graph=200, replays=5):
    """Cross-check: per batch size, `per_graph` back-to-back calls cycling the weight ring
    captured into one HIP graph on a stream of its own (the calls are built for that
    stream); each replay timed with one event pair.  Returns the median, min and max us
    per projection over `replays` replays, after checking that every replay leaves the
    same outputs as an eager call."""
    out = {}
    gs = torch.cuda.Stream()
    with torch.cuda.stream(gs):
        L2 = Launcher(torch, sg)  # its launches go to gs
    for M in m_list:
        calls = [make_call(L2, M, r) for r in range(R)]
        with torch.cuda.stream(gs):
            calls[0]()
        torch.cuda.synchronize()
        eager = y32[M].clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=gs):
            for i in range(per_graph):
                calls[(i + 1) % R]()  # ends on copy (per_graph % R), equal to copy 0
        times = []
        for _ in range(replays):
            y32[M].fill_(float("nan"))
            torch.cuda.synchronize()
            start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(gs):
                start.record()
                g.replay()
                stop.record()
            torch.cuda.synchronize()
            times.append(1e3 * start.elapsed_time(stop) / per_graph)
            if not torch.equal(y32[M], eager):
                raise RuntimeError(f"graph replay at M={M} differs from the eager call")
        times.sort()
        out[str(M)] = {"median_us": round(times[len(times) // 2], 3), "min_us": round(times[0], 3),
                       "max_us": round(times[-1], 3)}
        del g
    return out


def graph_us(torch, sg, make_calls, out, per_graph=200, replays=5):
    """Median us per call of `per_graph` back-to-back calls captured in one HIP graph on a
    stream of its own (make_calls(launcher) builds the calls for that stream's launcher),
    after checking that every replay leaves `out` as an eager call does."""
    gs = torch.cuda.Stream()
    with torch.cuda.stream(gs):
        L2 = Launcher(torch, sg)
    calls = make_calls(L2)
    with torch.cuda.stream(gs):
        calls[0]()
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=gs):
        for i in range(per_graph):
            calls[(i + 1) % len(calls)]()
    times = []
    for _ in range(replays):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(gs):
            start.record()
            g.replay()
            stop.record()
        torch.cuda.synchronize()
        times.append(1e3 * start.elapsed_time(stop) / per_graph)
        if not torch.equal(out, eager):
            raise RuntimeError("graph replay differs from the eager call")
    del g
    times.sort()
    return round(times[len(times) // 2], 3)


class SweepJournal:
    """The sweep's rows as JSON lines: every finished section appends its rows and then a
    {"section_done": name} line, so a killed sweep run again with the same file skips the
    sections already there (their rows are reused) and measures the rest."""

    def __init__(self, path):
        self.path = path
        self.done = {}
        pending = []
        if os.path.exists(path):
            with open(path) as f:
                for line in f:
                    line = line.strip()
                    if not line:
                        continue
                    try:
                        obj = json.loads(line)
                    except json.JSONDecodeError:
                        break  # a line cut short by the kill: the rest is measured again
                    if "section_done" in obj:
                        self.done[obj["section_done"]] = pending
                        pending = []
                    else:
                        pending.append(obj)
            # rewrite the file with the complete sections only
            with open(path, "w") as f:
                for name, rows in self.done.items():
                    for r in rows:
                        f.write(json.dumps(r) + "\n")
                    f.write(json.dumps({"section_done": name}) + "\n")

    def write(self, name, rows):
        with open(self.path, "a") as f:
            for r in rows:
                f.write(json.dumps(r) + "\n")
            f.write(json.dumps({"section_done": name}) + "\n")
            f.flush()
            os.fsync(f.fileno())
        self.done[name] = list(rows)


def sweep(torch, sg, si, L, cyc, reps=40, journal=None):
    dev = "cuda"
    rows = []

    def record(name, M, N, K, plan_desc, ms, nbytes):
        us = 1e3 * ms
        rows.append({"workload": name, "M": M, "N": N, "K": K, "plan": plan_desc,
                     "us": round(us, 3), "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
                     "pct_peak": round(100.0 * nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 1)})

    def plan_desc(p):
        return f"{sg.KERNEL_NAMES[p.kernel]} S={p.split_k}"

    def run_section(name, fn):
        # with --jsonl, a section already in the file is taken from it (a killed sweep
        # resumes there); a measured one is appended to it as soon as it is done
        if journal is not None and name in journal.done:
            rows.extend(journal.done[name])
            log(f"sweep: section '{name}' taken from {journal.path}")
            return
        start = len(rows)
        fn()
        if journal is not None:
            journal.write(name, rows[start:])

    def section_0():
        # single decode projection M=1, K=N=1024 (launch-bound)
        N = K = 1024
        x = si.normal_bf16((1, K), 0.02, si.seed_for(1, si.TAG_X), dev)
        ring = ring_copies(torch, si.normal_bf16((N, K), 0.02, si.seed_for(1, si.TAG_W), dev))
        p = sg.skinny_gemm_plan(1, N, K)
        y = torch.empty((1, N), device=dev)
        per = timed_calls(torch, [L.projection(p, x, w, y, None) for w in ring], 512, cyc)
        record("single 1024x1024", 1, N, K, plan_desc(p), per, proj_bytes(1, N, K, bf16=False))
        del ring

    run_section("single 1024x1024", section_0)

    def section_1():
        # small batch M in {1,2}, K=7168, N=8192, fp32 + bf16 out
        N, K = 8192, 7168
        ring = ring_copies(torch, si.normal_bf16((N, K), 0.02, si.seed_for(2, si.TAG_W), dev))
        for M in (1, 2):
            x = si.normal_bf16((M, K), 1.0, si.seed_for(2, si.TAG_X) + M, dev)
            p = sg.skinny_gemm_plan(M, N, K)
            y32, y16 = torch.empty((M, N), device=dev), torch.empty((M, N), device=dev, dtype=torch.bfloat16)
            per = timed_calls(torch, [L.projection(p, x, w, y32, y16) for w in ring], reps, cyc)
            record("small-batch 8192x7168", M, N, K, plan_desc(p), per, proj_bytes(M, N, K))
        # the same matrix at larger decode batches (the planner's kernel at each M)
        for M in (4, 8, 16, 64):
            x = si.normal_bf16((M, K), 1.0, si.seed_for(2, si.TAG_X) + M, dev)
            p = sg.skinny_gemm_plan(M, N, K)
            y32, y16 = torch.empty((M, N), device=dev), torch.empty((M, N), device=dev, dtype=torch.bfloat16)
            ws = torch.empty(max(p.workspace_bytes, 256), dtype=torch.uint8, device=dev)
            per = timed_calls(torch, [L.projection(p, x, w, y32, y16, ws) for w in ring], reps, cyc)
            record("8192x7168, larger batch", M, N, K, plan_desc(p), per, proj_bytes(M, N, K))

        # side-stream weight prefetch on the same ring: the read of one 117 MB matrix alone, and
        # what it buys the projection after it -- prefetch then project the same matrix (its
        # weights now in the Infinity Cache) against prefetch one matrix and project another
        # that was last read two pairs earlier (cold).  Both pair streams run the same kernels;
        # their difference is the cold-minus-warm projection time.
        nbytes = N * K * 2
        sp = L.sp

        def pf(w):
            def go():
                st = L.c.skinny_gemm_prefetch(w.data_ptr(), nbytes, sp)
                if st:
                    raise RuntimeError(sg.skinny_gemm_status_str(st))
            return go
        x = si.normal_bf16((1, K), 1.0, si.seed_for(2, si.TAG_X) + 1, dev)
        p = sg.skinny_gemm_plan(1, N, K)
        y32, y16 = torch.empty((1, N), device=dev), torch.empty((1, N), device=dev, dtype=torch.bfloat16)
        proj = [L.projection(p, x, w, y32, y16) for w in ring]
        n = len(ring)
        alone = timed_calls(torch, [pf(w) for w in ring], reps, cyc)
        same = timed_calls(torch, [c for i in range(n) for c in (pf(ring[i]), proj[i])], 2 * reps, cyc)
        other = timed_calls(torch, [c for i in range(n) for c in (pf(ring[(i + 2) % n]), proj[i])],
                            2 * reps, cyc)
        us = 1e3 * alone
        rows.append({"workload": "prefetch 8192x7168 (one 117 MB matrix)", "M": 1, "N": N, "K": K,
                     "plan": "prefetch", "us": round(us, 3),
                     "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
                     "pct_peak": round(100.0 * nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 1),
                     "projection_after_prefetch_us": round(2e3 * same - us, 3),
                     "projection_cold_us": round(2e3 * other - us, 3)})
        del ring

    run_section("8192x7168", section_1)

    def section_2():
        # split-K sweep M in {4..64}, K=7168, N=4096, fp32 out
        N, K = 4096, 7168
        ring = ring_copies(torch, si.normal_bf16((N, K), 0.02, si.seed_for(3, si.TAG_W), dev))
        # first, this matrix read with no arithmetic (the read probe on the M = 1 plan's shape)
        p1 = sg.skinny_gemm_plan(1, N, K)
        per = timed_calls(torch, [L.read_probe(w, p1.tile_n, p1.grid) for w in ring], reps, cyc)
        record("read probe 4096x7168 (weights only)", 0, N, K,
               f"read_probe rows_per_iter={p1.tile_n} grid={p1.grid}", per, N * K * 2)
        for M in (3, 4, 8, 12, 16, 32, 48, 64):
            x = si.normal_bf16((M, K), 1.0, si.seed_for(3, si.TAG_X) + M, dev)
            p = sg.skinny_gemm_plan(M, N, K)
            y32 = torch.empty((M, N), device=dev)
            ws = torch.empty(max(p.workspace_bytes, 256), dtype=torch.uint8, device=dev)
            per = timed_calls(torch, [L.projection(p, x, w, y32, None, ws) for w in ring], reps, cyc)
            record("split-K 4096x7168", M, N, K, plan_desc(p), per, proj_bytes(M, N, K, bf16=False))
            if M in (4, 16, 32, 64):  # also as 200 calls in one HIP graph (one or two launches each)
                rows[-1]["us_graph"] = graph_us(
                    torch, sg, lambda L2, p=p, x=x, y32=y32, ws=ws:
                    [L2.projection(p, x, w, y32, None, ws) for w in ring], y32)
        # the same shapes at each split factor the workload names, S in {2, 4, 8, 16} (vector ALU
        # below 8 rows, matrix cores from 8; the library picks the reduction and the row tiling)
        for M in (4, 8, 16, 32, 64):
            x = si.normal_bf16((M, K), 1.0, si.seed_for(3, si.TAG_X) + M, dev)
            y32 = torch.empty((M, N), device=dev)
            kernel = sg.SG_KERNEL_SPLITK_VALU if M < 8 else sg.SG_KERNEL_SPLITK_MFMA
            for S in (2, 4, 8, 16):
                try:
                    p = sg.skinny_gemm_plan_force(M, N, K, kernel, S)
                except sg.SkinnyGemmError:
                    continue
                ws = torch.empty(max(p.workspace_bytes, 256), dtype=torch.uint8, device=dev)
                per = timed_calls(torch, [L.projection(p, x, w, y32, None, ws) for w in ring], reps,
                                  cyc)
                record("split-K 4096x7168, forced split", M, N, K,
                       f"{plan_desc(p)} tile={p.tile_n} two_pass={p.two_pass}", per,
                       proj_bytes(M, N, K, bf16=False))
        del ring

    run_section("split-K 4096x7168", section_2)

    def section_3():
        # fused output projection + residual, K=8192, N=7168, bf16 out
        N, K = 7168, 8192
        ring = ring_copies(torch, si.normal_bf16((N, K), 0.02, si.seed_for(4, si.TAG_W), dev))
        for M in (1, 8, 64):
            x = si.normal_bf16((M, K), 1.0, si.seed_for(4, si.TAG_X) + M, dev)
            r = si.normal_bf16((M, N), 1.0, si.seed_for(4, si.TAG_R) + M, dev)
            p = sg.skinny_gemm_plan(M, N, K)
            o16 = torch.empty((M, N), device=dev, dtype=torch.bfloat16)
            ws = torch.empty(max(p.workspace_bytes, 256), dtype=torch.uint8, device=dev)
            per = timed_calls(torch, [L.residual(p, x, w, r, o16, None, ws) for w in ring], reps, cyc)
            record("residual 7168x8192", M, N, K, plan_desc(p), per,
                   proj_bytes(M, N, K, f32=False, residual=True))
            rows[-1]["us_graph"] = graph_us(
                torch, sg, lambda L2, p=p, x=x, r=r, o16=o16, ws=ws:
                [L2.residual(p, x, w, r, o16, None, ws) for w in ring], o16)
        del ring
        torch.cuda.empty_cache()

    run_section("residual 7168x8192", section_3)

    def section_4():
        # MXFP4 weights (e2m1 codes + e8m0 block scales): the same shapes at a quarter of the
        # weight bytes; a ring of code/scale copies larger than 2 x MALL per shape
        c = L.c
        for label, Ms, N, K, residual in (("mxfp4 8192x7168", (1, 2, 16, 64), 8192, 7168, False),
                                          ("mxfp4 4096x7168", (4, 8, 16, 32, 64), 4096, 7168, False),
                                          ("mxfp4 residual 7168x8192", (1, 8, 64), 7168, 8192, True)):
            codes, scales = si.mxfp4_weights(N, K, si.seed_for(6, si.TAG_W) + N, dev)
            per_copy = codes.numel() + scales.numel()
            copies = max(1, math.ceil(RING_MIN_BYTES / per_copy))
            ring = [(codes, scales)] + [(codes.clone(), scales.clone()) for _ in range(copies - 1)]
            for M in Ms:
                x = si.normal_bf16((M, K), 1.0, si.seed_for(6, si.TAG_X) + M, dev)
                r = si.normal_bf16((M, N), 1.0, si.seed_for(6, si.TAG_R) + M, dev) if residual else None
                y32 = None if residual else torch.empty((M, N), device=dev)
                y16 = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

                wsb = sg.skinny_gemm_mxfp4_workspace(M, N, K)
                ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)

                def mx(cw, sw, x=x, r=r, y32=y32, y16=y16, M=M, N=N, K=K, ws=ws, wsb=wsb):
                    args = (M, N, K, x.data_ptr(), cw.data_ptr(), sw.data_ptr(),
                            r.data_ptr() if r is not None else None,
                            y32.data_ptr() if y32 is not None else None, y16.data_ptr(),
                            ws.data_ptr(), wsb, L.sp)

                    def go():
                        st = c.skinny_gemm_mxfp4(*args)
                        if st:
                            raise RuntimeError(sg.skinny_gemm_status_str(st))
                    return go
                per = timed_calls(torch, [mx(cw, sw) for cw, sw in ring], reps, cyc)
                nbytes = N * K // 2 + N * K // 32 + M * K * 2 + M * N * 2 * (2 if residual else 1) + \
                    (0 if residual else M * N * 4)
                us = 1e3 * per
                gbs = nbytes / (per * 1e-3) / 1e9
                rows.append({"workload": label, "M": M, "N": N, "K": K,
                             "plan": lowp_plan_label("mxfp4", M, N, wsb),
                             "us": round(us, 3), "GBps": round(gbs, 1),
                             "pct_peak": round(100 * gbs / HBM_PEAK_GBS, 1)})
            del ring
        torch.cuda.empty_cache()

    run_section("mxfp4", section_4)

    def section_5():
        c = L.c
        # FP8 e4m3 weights with 128 x 128 fp32 block scales: half the bf16 weight bytes; a ring
        # of code/scale copies larger than 2 x MALL per shape
        for label, Ms, N, K, residual in (("fp8 8192x7168", (1, 2, 16, 64), 8192, 7168, False),
                                          ("fp8 4096x7168", (4, 8, 16, 32, 64), 4096, 7168, False),
                                          ("fp8 residual 7168x8192", (1, 64), 7168, 8192, True)):
            codes, scales = si.fp8_weights(N, K, si.seed_for(7, si.TAG_W) + N, dev)
            per_copy = codes.numel() + scales.numel() * 4
            copies = max(1, math.ceil(RING_MIN_BYTES / per_copy))
            ring = [(codes, scales)] + [(codes.clone(), scales.clone()) for _ in range(copies - 1)]
            for M in Ms:
                x = si.normal_bf16((M, K), 1.0, si.seed_for(7, si.TAG_X) + M, dev)
                r = si.normal_bf16((M, N), 1.0, si.seed_for(7, si.TAG_R) + M, dev) if residual else None
                y32 = None if residual else torch.empty((M, N), device=dev)
                y16 = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

                wsb = sg.skinny_gemm_fp8_workspace(M, N, K)
                ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)

                def f8(cw, sw, x=x, r=r, y32=y32, y16=y16, M=M, N=N, K=K, ws=ws, wsb=wsb):
                    args = (M, N, K, x.data_ptr(), cw.data_ptr(), sw.data_ptr(),
                            r.data_ptr() if r is not None else None,
                            y32.data_ptr() if y32 is not None else None, y16.data_ptr(),
                            ws.data_ptr(), wsb, L.sp)

                    def go():
                        st = c.skinny_gemm_fp8(*args)
                        if st:
                            raise RuntimeError(sg.skinny_gemm_status_str(st))
                    return go
                per = timed_calls(torch, [f8(cw, sw) for cw, sw in ring], reps, cyc)
                nbytes = N * K + scales.numel() * 4 + M * K * 2 + M * N * 2 * (2 if residual else 1) + \
                    (0 if residual else M * N * 4)
                us = 1e3 * per
                gbs = nbytes / (per * 1e-3) / 1e9
                rows.append({"workload": label, "M": M, "N": N, "K": K,
                             "plan": lowp_plan_label("fp8", M, N, wsb),
                             "us": round(us, 3), "GBps": round(gbs, 1),
                             "pct_peak": round(100 * gbs / HBM_PEAK_GBS, 1)})
            del ring
        torch.cuda.empty_cache()

    run_section("fp8", section_5)

    def section_6():
        # router: scores y = x W_r^T (E=384 experts, K=7168, fp32) and their top-8 per token
        E, K, k = 384, 7168, 8
        Wr = si.normal_bf16((E, K), 0.02, si.seed_for(5, si.TAG_W) + 99, dev)
        ring = ring_copies(torch, Wr)
        c = L.c
        for T in (1, 16, 64):
            x = si.normal_bf16((T, K), 1.0, si.seed_for(5, si.TAG_X) + T, dev)
            p = sg.skinny_gemm_plan(T, E, K)
            scores = torch.empty((T, E), device=dev)
            ids = torch.empty((T, k), dtype=torch.int32, device=dev)
            ws = torch.empty(max(p.workspace_bytes, 256), dtype=torch.uint8, device=dev)

            def router(proj, scores=scores, ids=ids, T=T):
                def go():
                    proj()
                    st = c.skinny_gemm_router_topk(scores.data_ptr(), T, E, k, ids.data_ptr(), None,
                                                   L.sp)
                    if st:
                        raise RuntimeError(sg.skinny_gemm_status_str(st))
                return go
            per = timed_calls(torch, [router(L.projection(p, x, w, scores, None, ws)) for w in ring],
                              reps, cyc)
            nbytes = proj_bytes(T, E, K, bf16=False) + T * E * 4 + T * k * 4
            rows.append({"workload": "router top-8 E=384 K=7168", "M": T, "N": E, "K": K,
                         "plan": f"{plan_desc(p)}+router_topk", "us": round(1e3 * per, 3),
                         "GBps": round(nbytes / (per * 1e-3) / 1e9, 1),
                         "pct_peak": round(100.0 * nbytes / (per * 1e-3) / 1e9 / HBM_PEAK_GBS, 1)})
        del ring, Wr

    run_section("router", section_6)

    def section_7():
        # MoE grouped: E=384 experts of N=2048 x K=7168, 8 distinct experts per token,
        # a ring of 8 routing tables per batch size
        E, N, K, topk = 384, 2048, 7168, 8
        W = si.normal_bf16((E, N, K), 0.02, si.seed_for(5, si.TAG_W) + 100, dev)
        for T in (1, 16, 64):
            x = si.normal_bf16((T, K), 1.0, si.seed_for(5, si.TAG_X) + T, dev)
            tables = [si.routing_table(T, E, topk, si.seed_for(5, si.TAG_ROUTING) + 10 * i + 1000 * T)
                      for i in range(8)]
            out = torch.empty((T, topk, N), device=dev)
            ws = torch.empty(sg.grouped_skinny_gemm_workspace(T, E, topk, N, K), dtype=torch.uint8,
                             device=dev)
            ids_dev = [t.to(dev) for t in tables]
            per = timed_calls(torch, [L.grouped(x, W, ids, out, ws) for ids in ids_dev],
                                 8 * max(1, reps // 32), cyc)
            distinct = [len(set(t.view(-1).tolist())) for t in tables]
            # the timed calls cycle the tables evenly (reps is a multiple of 8)
            nbytes = sum(d * N * K * 2 + T * K * 2 + T * topk * N * 4 + T * topk * 4
                         for d in distinct) / len(distinct)
            us = 1e3 * per
            gbs = nbytes / (per * 1e-3) / 1e9
            rows.append({"workload": "MoE grouped E=384 2048x7168 top8", "M": T, "N": N, "K": K,
                         "plan": "fused table+grouped", "us": round(us, 3), "GBps": round(gbs, 1),
                         "pct_peak": round(100 * gbs / HBM_PEAK_GBS, 1),
                         "distinct_experts_mean": round(sum(distinct) / len(distinct), 1)})

        # one MoE decode step: router scores + top-8 + table + grouped routed experts, and a
        # shared expert of the same shape as one routed expert (N=2048, K=7168): fused into the
        # router's GEMM, on a side stream overlapping the routing, or serial.  Rings: inputs (8)
        # and [router; shared expert] weight pairs (> 2 x MALL).
        Wrs = torch.cat([si.normal_bf16((E, K), 0.02, si.seed_for(5, si.TAG_W) + 99, dev),
                         si.normal_bf16((N, K), 0.02, si.seed_for(5, si.TAG_W) + 98, dev)])
        ring_rs = ring_copies(torch, Wrs)
        for T in (1, 16, 64):
            xs = [si.normal_bf16((T, K), 1.0, si.seed_for(5, si.TAG_X) + 100 * T + i, dev)
                  for i in range(8)]
            n_calls = max(len(ring_rs), len(xs))
            combos = [(xs[i % len(xs)], ring_rs[i % len(ring_rs)][:E], ring_rs[i % len(ring_rs)][E:])
                      for i in range(n_calls)]
            outs = (torch.empty((T, topk), dtype=torch.int32, device=dev),
                    torch.empty((T, E + N), device=dev), torch.empty((T, topk, N), device=dev),
                    torch.empty((T, N), device=dev))
            ws = torch.empty(sg.skinny_moe_step_workspace(T, K, E, topk, N, N), dtype=torch.uint8,
                             device=dev)
            distinct = []
            for x, wr, wsh in combos:  # the experts each call routes to (same inputs as timed)
                L.moe_step(x, wr, W, wsh, topk, outs, ws, "serial")()
                torch.cuda.synchronize()
                distinct.append(len(set(outs[0].view(-1).tolist())))
            nbytes = sum(d * N * K * 2 for d in distinct) / len(distinct) + \
                proj_bytes(T, E, K, bf16=False) + proj_bytes(T, N, K, bf16=False) - T * K * 2 + \
                T * topk * N * 4 + T * topk * 4
            per = {}
            launches = {}
            for mode in ("serial", "side_stream", "fused", "shared_in_routed"):
                calls = [L.moe_step(x, wr, W, wsh, topk, outs, ws, mode) for x, wr, wsh in combos]
                before = sg.skinny_gemm_get_counters()
                calls[0]()
                torch.cuda.synchronize()
                launches[mode] = sum(a - b for a, b in zip(sg.skinny_gemm_get_counters(), before))
                per[mode] = timed_calls(torch, calls, n_calls, cyc)
            gbs = nbytes / (per["fused"] * 1e-3) / 1e9
            rows.append({"workload": "MoE step E=384 top8 2048x7168 + shared expert", "M": T,
                         "N": N, "K": K, "plan": "router+shared fused GEMM, top8, table, grouped",
                         "us": round(1e3 * per["fused"], 3),
                         "us_side_stream": round(1e3 * per["side_stream"], 3),
                         "us_serial": round(1e3 * per["serial"], 3),
                         "us_shared_in_routed": round(1e3 * per["shared_in_routed"], 3),
                         "launches_per_step": launches["fused"],
                         "launches_shared_in_routed": launches["shared_in_routed"],
                         "GBps": round(gbs, 1), "pct_peak": round(100 * gbs / HBM_PEAK_GBS, 1),
                         "distinct_experts_mean": round(sum(distinct) / len(distinct), 1)})
        del W, Wrs, ring_rs
        torch.cuda.empty_cache()

    run_section("moe", section_7)

    return rows


def side_stream_cu_mask(torch, sg, si, L, cyc, cus, Ts=(1, 4, 16), reps=5):
    """The MoE step with the shared expert on a side stream restricted to the first `cus`
    compute units (hipExtStreamCreateWithCUMask, default priority), against the
    library's fused, serial and side-stream placements on unmasked streams.  Median us over
    reps rounds."""
    import statistics
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipExtStreamCreateWithCUMask.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint32,
                                                 ctypes.POINTER(ctypes.c_uint32)]
    hip.hipStreamDestroy.argtypes = [ctypes.c_void_p]
    dev = "cuda"
    E, N, K, topk = 384, 2048, 7168, 8
    W = si.normal_bf16((E, N, K), 0.02, si.seed_for(5, si.TAG_W), dev)
    Wrs = torch.cat([si.normal_bf16((E, K), 0.02, si.seed_for(5, si.TAG_W) + 99, dev),
                     si.normal_bf16((N, K), 0.02, si.seed_for(5, si.TAG_W) + 98, dev)])
    ring_rs = ring_copies(torch, Wrs)
    fork, join = torch.cuda.Event(), torch.cuda.Event()
    cur = torch.cuda.current_stream()
    fork.record(cur)  # torch creates the hipEvent_t at its first record
    join.record(cur)
    words = (ctypes.c_uint32 * 8)()
    for b in range(cus):
        words[b // 32] |= 1 << (b % 32)
    side = ctypes.c_void_p()
    st = hip.hipExtStreamCreateWithCUMask(ctypes.byref(side), 8, words)
    if st != 0:
        raise RuntimeError(f"hipExtStreamCreateWithCUMask: error {st}")
    rows = []
    try:
        for T in Ts:
            xs = [si.normal_bf16((T, K), 1.0, si.seed_for(5, si.TAG_X) + 100 * T + i, dev)
                  for i in range(8)]
            n_calls = max(len(ring_rs), len(xs))
            combos = [(xs[i % len(xs)], ring_rs[i % len(ring_rs)][:E],
                       ring_rs[i % len(ring_rs)][E:]) for i in range(n_calls)]
            outs = (torch.empty((T, topk), dtype=torch.int32, device=dev),
                    torch.empty((T, E + N), device=dev), torch.empty((T, topk, N), device=dev),
                    torch.empty((T, N), device=dev))
            ws = torch.empty(sg.skinny_moe_step_workspace(T, K, E, topk, N, N),
                             dtype=torch.uint8, device=dev)
            variants = {m: [L.moe_step(x, wr, W, wsh, topk, outs, ws, m) for x, wr, wsh in combos]
                        for m in ("fused", "serial", "side_stream")}
            steps = []
            for x, wr, wsh in combos:
                steps.append(sg.SgMoeStep(x.data_ptr(), wr.data_ptr(), W.data_ptr(), wsh.data_ptr(),
                                          outs[1].data_ptr(), outs[0].data_ptr(), None,
                                          outs[2].data_ptr(), outs[3].data_ptr(),
                                          T, K, E, topk, N, N, 0))

            def masked(step):
                ref = ctypes.byref(step)

                def go():
                    st = L.c.skinny_moe_step(ref, ws.data_ptr(), ws.numel(), L.sp, side,
                                             fork.cuda_event, join.cuda_event)
                    if st:
                        raise RuntimeError(sg.skinny_gemm_status_str(st))
                return go
            variants["side_stream_cu_masked"] = [masked(step) for step in steps]
            times = {k: [] for k in variants}
            for calls in variants.values():
                calls[0]()
            torch.cuda.synchronize()
            for _ in range(reps):
                for k, calls in variants.items():
                    times[k].append(1e3 * timed_calls(torch, calls, n_calls, cyc))
            rows.append({"T": T, "cus": cus,
                         **{f"us_{k}": round(statistics.median(v), 2) for k, v in times.items()}})
            log(json.dumps(rows[-1]))
    finally:
        torch.cuda.synchronize()
        hip.hipStreamDestroy(side)
    return rows


# --------------------------------------------------------------------------- CPU baseline


def _host_threads() -> int:
    """Worker threads for the oracle: the cores this process may run on, capped by
    OMP_NUM_THREADS when the host sets it (the share of the host one GPU gets)."""
    n = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_rows(o, pool, threads, xb, Wb):
    """The oracle's projection over row slices of W, one slice per thread (the C call
    releases the GIL, so the slices run in parallel); the oracle itself is unchanged."""
    import numpy as np
    N = Wb.shape[0]
    cuts = sorted({int(round(N * i / threads)) for i in range(threads + 1)})
    futs = [pool.submit(o.projection, xb, Wb[a:b], False) for a, b in zip(cuts, cuts[1:])]
    return np.concatenate([f.result() for f in futs], axis=1)


def _time_loop(fn, budget_s):
    """Calls fn until budget_s has passed (at least once); returns (calls, seconds)."""
    calls, t0 = 0, time.perf_counter()
    while True:
        fn()
        calls += 1
        if time.perf_counter() - t0 >= budget_s:
            return calls, time.perf_counter() - t0


def cpu_baseline(si, inputs, budget_s=8.0, sample_rows=512):
    """The fp64 oracle, as it stands, on this host: single-threaded and over row slices
    on every available core, on full M = 1 and M = 2 projections of the headline
    workload; then per workload configuration (full projections on all cores,
    single-threaded on a row sample scaled to the full matrix)."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import oracle

    o = oracle.Oracle()
    threads = _host_threads()
    x, W0 = inputs
    Wb = si.bits(W0)
    xb = {M: si.bits(x[M]) for M in M_LIST}
    step_bytes = sum(proj_bytes(M, N_MAIN, K_MAIN) for M in M_LIST)
    with ThreadPoolExecutor(max_workers=threads) as pool:
        n1, t1 = _time_loop(lambda: [o.projection(xb[M], Wb, False) for M in M_LIST],
                            budget_s / 2)
        nt, tt = _time_loop(lambda: [_oracle_rows(o, pool, threads, xb[M], Wb) for M in M_LIST],
                            budget_s / 2)
        single_gbs = step_bytes * n1 / t1 / 1e9
        multi_gbs = step_bytes * nt / tt / 1e9

        def host_bf16(shape, sigma, seed):
            return si.bits(si.normal_bf16(shape, sigma, seed, "cpu"))

        per_config = []

        def add(workload, M, N, K, nbytes, full_fn, sample_fn, rows):
            # all cores on the full projection; one core on `rows` rows, scaled to N
            n_f, t_f = _time_loop(full_fn, 0.0)
            n_s, t_s = _time_loop(sample_fn, 0.0)
            ms_all = 1e3 * t_f / n_f
            ms_one = 1e3 * t_s / n_s * N / rows
            per_config.append({
                "workload": workload, "M": M, "N": N, "K": K,
                "ms_single": round(ms_one, 3), "GBps_single": round(nbytes / ms_one / 1e6, 4),
                "ms_threads": round(ms_all, 3), "GBps_threads": round(nbytes / ms_all / 1e6, 4),
                "single_sample_rows": rows})

        # single decode projection 1024 x 1024 (every row in both legs)
        x1, W1 = host_bf16((1, 1024), 0.02, 1000), host_bf16((1024, 1024), 0.02, 1001)
        add("single decode projection", 1, 1024, 1024, proj_bytes(1, 1024, 1024, bf16=False),
            lambda: _oracle_rows(o, pool, threads, x1, W1), lambda: o.projection(x1, W1, False),
            1024)
        # small batch 8192 x 7168 (the headline legs above, per batch size)
        for M in M_LIST:
            nb = proj_bytes(M, N_MAIN, K_MAIN)
            add("small batch (headline)", M, N_MAIN, K_MAIN, nb,
                lambda M=M: _oracle_rows(o, pool, threads, xb[M], Wb),
                lambda M=M: o.projection(xb[M], Wb[:sample_rows], False), sample_rows)
        # split-K sweep 4096 x 7168
        W3 = host_bf16((4096, 7168), 0.02, 3001)
        for M in (4, 8, 16, 32, 64):
            x3 = host_bf16((M, 7168), 1.0, 3000 + M)
            add("split-K sweep", M, 4096, 7168, proj_bytes(M, 4096, 7168, bf16=False),
                lambda x3=x3: _oracle_rows(o, pool, threads, x3, W3),
                lambda x3=x3: o.projection(x3, W3[:sample_rows], False), sample_rows)
        del W3
        # fused residual 7168 x 8192 (projection, then the residual add)
        W4 = host_bf16((7168, 8192), 0.02, 4001)
        for M in (1, 8, 64):
            x4, r4 = host_bf16((M, 8192), 1.0, 4000 + M), host_bf16((M, 7168), 1.0, 4002 + M)
            add("fused residual", M, 7168, 8192,
                proj_bytes(M, 7168, 8192, f32=False, residual=True),
                lambda x4=x4, r4=r4: o.residual(r4, _oracle_rows(o, pool, threads, x4, W4)),
                lambda x4=x4, r4=r4: o.residual(r4[:, :sample_rows],
                                                o.projection(x4, W4[:sample_rows], False)),
                sample_rows)
        del W4
        # MoE grouped, one token routed to 8 experts of 2048 x 7168: the 8 experts'
        # weights only (the other 376 are never read); all cores take one pair each
        We = host_bf16((8, 2048, 7168), 0.02, 5100)
        x5 = host_bf16((1, 7168), 1.0, 5000)
        ids = np.arange(8, dtype=np.int32).reshape(1, 8)
        nb5 = 8 * 2048 * 7168 * 2 + 7168 * 2 + 8 * 2048 * 4
        add("MoE grouped E=384 top8, T=1", 1, 2048, 7168, nb5,
            lambda: [f.result() for f in [pool.submit(o.grouped, x5, We, ids[:, j:j + 1], False)
                                          for j in range(8)]],
            lambda: o.grouped(x5, We, ids[:, :1], False), 2048 // 8)
        del We
    return {"value": round(multi_gbs, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "single": {"value": round(single_gbs, 4), "unit": "GB/s", "cores": 1},
            "threads": threads,
            "host_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "cpu_model": _cpu_model(),
            "sample": f"headline: {nt} full steps (M=1 and M=2 projections, K=7168, N=8192) over "
                      f"{threads} threads (row slices of W, one fp64 C oracle call each) in "
                      f"{tt:.1f} s; single-threaded {n1} steps in {t1:.1f} s. per_config: full "
                      f"projections on {threads} threads; single-threaded time measured on the "
                      f"first {sample_rows} rows of W (MoE: one of the 8 pairs) and scaled to "
                      f"the full matrix; MoE at T=1 only (larger T needs the whole 11 GB "
                      f"expert set on the host)",
            "per_config": per_config}


# --------------------------------------------------------------------------- traffic (PMC)


def read_traffic():
    """HBM traffic per GEMV launch from the committed rocprofv3 counter summary, or None
    when the summary is missing or the kernel source changed since it was taken."""
    if not os.path.exists(PROFILE_TRAFFIC):
        return None
    vals = {}
    with open(PROFILE_TRAFFIC) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


COPY_BYTES = 1 << 30          # the calibration copy reads and writes this many bytes
COPY_KERNEL_TAG = "MulFunctor"  # torch.mul(src, 1.0, out=dst): a plain element-wise copy
COPY_GRID = COPY_BYTES // 16    # its launch: one thread per 4 floats
# the headline launches: rowstream_kernel<M, NCH, S, ITERS> with 14 loads a row,
# one wave a row and 4 rows a wave (8192 rows on 2048 waves, K = 7168)
GEMV_KERNEL_TAGS = ("rowstream_kernel<1, 14, 1, 4>", "rowstream_kernel<2, 14, 1, 4>")


def _pmc_dispatches(directory: str) -> list:
    """(kernel name, counter, grid size, value in KiB) per dispatch, from the rocprofv3
    counter_collection CSVs under directory."""
    rows = []
    for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            rows += list(csv.DictReader(f))
    if not rows:
        raise SystemExit(f"no counter_collection.csv under {directory}")
    per = {}
    for r in rows:
        key = (r["Kernel_Name"], r["Counter_Name"], int(r["Grid_Size"]), r["Dispatch_Id"])
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    return [(name, c, grid, v) for (name, c, grid, _), v in per.items()]


def summarize_pmc(fetch_dir: str, write_dir: str) -> None:
    """Print the HBM-traffic summary of the small-matrix kernel (committed under profiles/):
    FETCH_SIZE and WRITE_SIZE per dispatch, each scaled by what the same counter reads
    for the calibration copy of known size."""
    fetch, write = _pmc_dispatches(fetch_dir), _pmc_dispatches(write_dir)

    def pick(table, counter, tags, calibration=False):
        hits = [(name, grid, v) for name, c, grid, v in table
                if c == counter and any(t in name for t in tags)]
        if calibration:  # the calibration copy: its kernel at exactly its launch size
            hits = [h for h in hits if h[1] == COPY_GRID]
        if not hits:
            raise SystemExit(f"no {counter} samples for {tags}")
        return (sum(v for _, _, v in hits) / len(hits), len(hits),
                sorted({name[:80] for name, _, _ in hits}))

    cf, _, _ = pick(fetch, "FETCH_SIZE", (COPY_KERNEL_TAG,), calibration=True)
    cw, _, _ = pick(write, "WRITE_SIZE", (COPY_KERNEL_TAG,), calibration=True)
    gf, nf, names = pick(fetch, "FETCH_SIZE", GEMV_KERNEL_TAGS)
    gw, nw, _ = pick(write, "WRITE_SIZE", GEMV_KERNEL_TAGS)
    fetch_factor = cf * 1024 / COPY_BYTES
    write_factor = cw * 1024 / COPY_BYTES
    traffic = gf * 1024 / fetch_factor + gw * 1024 / write_factor
    algo = sum(proj_bytes(M, N_MAIN, K_MAIN) for M in M_LIST) / len(M_LIST)
    print("# HBM traffic of the small-matrix kernel (M=1 and M=2, K=7168, N=8192), per launch")
    print("# from two rocprofv3 --pmc passes over the benchmark (FETCH_SIZE, then WRITE_SIZE),")
    print("# each counter scaled by its reading for a 1 GiB element-wise copy (torch.mul, out=).")
    print("# commands (repository root):")
    print("#   rocprofv3 --pmc FETCH_SIZE -f csv -d OUT/pmc_fetch -o f -- python bench.py "
          "--steps 10 --warmup 2 --no-sweep --no-cpu-baseline --copy-calibration")
    print("#   rocprofv3 --pmc WRITE_SIZE -f csv -d OUT/pmc_write -o w -- python bench.py "
          "--steps 10 --warmup 2 --no-sweep --no-cpu-baseline --copy-calibration")
    print("#   python bench.py --summarize-pmc OUT/pmc_fetch OUT/pmc_write")
    print(f"kernels: {'; '.join(names)}")
    print(f"kernel_source_sha256: {kernel_source_hash()}")
    print(f"dispatches_fetch: {nf}")
    print(f"dispatches_write: {nw}")
    print(f"copy_fetch_kib_per_dispatch: {cf:.1f}")
    print(f"copy_write_kib_per_dispatch: {cw:.1f}")
    print(f"fetch_scale: {fetch_factor:.4f}")
    print(f"write_scale: {write_factor:.4f}")
    print(f"gemv_fetch_kib_per_dispatch: {gf:.1f}")
    print(f"gemv_write_kib_per_dispatch: {gw:.1f}")
    print(f"traffic_bytes_per_launch: {traffic:.0f}")
    print(f"algorithmic_bytes_per_launch: {algo:.0f}")
    print(f"traffic_over_algorithmic: {traffic / algo:.4f}")


def summarize_trace(directory: str, command: str) -> None:
    """Print a per-kernel duration table from a rocprofv3 --kernel-trace --stats run."""
    paths = glob.glob(os.path.join(directory, "**", "*kernel_stats.csv"), recursive=True)
    if not paths:
        raise SystemExit(f"no kernel_stats.csv under {directory}")
    with open(paths[0]) as f:
        rows = list(csv.DictReader(f))
    print("# rocprofv3 kernel trace, per-kernel durations (us)")
    print(f"# command (repository root): {command}")
    print(f"# {'calls':>6} {'avg':>9} {'min':>9} {'max':>9}  kernel")
    for r in rows:
        name = r["Name"]
        print(f"  {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.2f} {float(r['MinNs']) / 1e3:9.2f} "
              f"{float(r['MaxNs']) / 1e3:9.2f}  {name[:150]}")


# --------------------------------------------------------------------------- per-workload counters


def profile_workloads(torch, sg, si, L, manifest_path, reps=3):
    """A fixed sequence of the benchmark's workloads, reps calls each (on distinct
    weight copies), for rocprofv3 --pmc passes; writes the manifest that maps the
    library's kernel dispatches, in order, back to the workloads."""
    dev = "cuda"
    copy_calibration(torch)
    manifest = []

    def run(label, M, N, K, plan, calls, nbytes):
        before = sg.skinny_gemm_get_counters()
        for i in range(reps):
            calls[i % len(calls)]()
        torch.cuda.synchronize()
        after = sg.skinny_gemm_get_counters()
        launched = sum(a - b for a, b in zip(after, before))
        manifest.append({"workload": label, "M": M, "N": N, "K": K, "plan": plan, "calls": reps,
                         "dispatches": launched, "bytes_per_call": nbytes})
        log(f"profiled {label} M={M}: {launched} dispatches")

    def desc(p):
        return f"{sg.KERNEL_NAMES[p.kernel]} S={p.split_k} tile={p.tile_n}"

    shapes = [("small-batch 8192x7168", M, 8192, 7168, dict()) for M in (1, 2)]
    shapes += [("split-K 4096x7168", M, 4096, 7168, dict(bf16=False))
               for M in (3, 4, 8, 12, 16, 32, 48, 64)]
    shapes += [("residual 7168x8192", M, 7168, 8192, dict(f32=False, residual=True))
               for M in (1, 8, 64)]
    for label, M, N, K, kind in shapes:
        W0 = si.normal_bf16((N, K), 0.02, 11, dev)
        ring = [W0] + [W0.clone() for _ in range(reps - 1)]
        x = si.normal_bf16((M, K), 1.0, 12, dev)
        p = sg.skinny_gemm_plan(M, N, K)
        ws = torch.empty(max(p.workspace_bytes, 256), dtype=torch.uint8, device=dev)
        if kind.get("residual"):
            r = si.normal_bf16((M, N), 1.0, 13, dev)
            o16 = torch.empty((M, N), device=dev, dtype=torch.bfloat16)
            calls = [L.residual(p, x, w, r, o16, None, ws) for w in ring]
        else:
            y32 = torch.empty((M, N), device=dev)
            y16 = None if kind.get("bf16") is False else torch.empty((M, N), device=dev,
                                                                    dtype=torch.bfloat16)
            calls = [L.projection(p, x, w, y32, y16, ws) for w in ring]
        run(label, M, N, K, desc(p), calls, proj_bytes(M, N, K, **kind))
        del ring, W0
        torch.cuda.empty_cache()
    # side-stream prefetch of one 117 MB matrix
    N, K = 8192, 7168
    W0 = si.normal_bf16((N, K), 0.02, 11, dev)
    ring = [W0] + [W0.clone() for _ in range(reps - 1)]
    run("prefetch 8192x7168", 1, N, K, "prefetch",
        [(lambda w=w: sg.skinny_gemm_prefetch(w)) for w in ring], N * K * 2)
    del ring, W0
    torch.cuda.empty_cache()
    E, N, K, topk = 384, 2048, 7168, 8
    W = si.normal_bf16((E, N, K), 0.02, 14, dev)
    for T in (1, 16, 64):
        x = si.normal_bf16((T, K), 1.0, 15, dev)
        ids = si.routing_table(T, E, topk, 16 + T)
        out = torch.empty((T, topk, N), device=dev)
        ws = torch.empty(sg.grouped_skinny_gemm_workspace(T, E, topk, N, K), dtype=torch.uint8,
                         device=dev)
        distinct = len(set(ids.view(-1).tolist()))
        nbytes = distinct * N * K * 2 + T * K * 2 + T * topk * N * 4 + T * topk * 4
        run("MoE grouped E=384 2048x7168 top8", T, N, K, "moe_table+grouped",
            [L.grouped(x, W, ids.to(dev), out, ws)], nbytes)
    del W
    torch.cuda.empty_cache()
    # MXFP4 weights
    for label, Ms, N, K in (("mxfp4 8192x7168", (1, 2, 16), 8192, 7168),
                            ("mxfp4 4096x7168", (4, 8, 16, 64), 4096, 7168)):
        codes, scales = si.mxfp4_weights(N, K, 17, dev)
        ring = [(codes, scales)] + [(codes.clone(), scales.clone()) for _ in range(reps - 1)]
        for M in Ms:
            x = si.normal_bf16((M, K), 1.0, 18, dev)
            y32 = torch.empty((M, N), device=dev)
            y16 = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            ws = torch.empty(max(sg.skinny_gemm_mxfp4_workspace(M, N, K), 256),
                             dtype=torch.uint8, device=dev)

            def mx(cw, sw, x=x, y32=y32, y16=y16, ws=ws):
                return lambda: sg.skinny_gemm_mxfp4(x, cw, sw, y_f32=y32, y_bf16=y16, workspace=ws)
            nbytes = N * K // 2 + N * K // 32 + M * K * 2 + M * N * 6
            run(label, M, N, K, lowp_plan_label("mxfp4", M, N, 0),
                [mx(cw, sw) for cw, sw in ring], nbytes)
        del ring
    # FP8 weights (e4m3 codes, 128 x 128 block scales)
    for label, Ms, N, K in (("fp8 8192x7168", (1, 2, 16), 8192, 7168),
                            ("fp8 4096x7168", (4, 8, 16, 64), 4096, 7168)):
        codes, scales = si.fp8_weights(N, K, 21, dev)
        ring = [(codes, scales)] + [(codes.clone(), scales.clone()) for _ in range(reps - 1)]
        for M in Ms:
            x = si.normal_bf16((M, K), 1.0, 22, dev)
            y32 = torch.empty((M, N), device=dev)
            y16 = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            ws = torch.empty(max(sg.skinny_gemm_fp8_workspace(M, N, K), 256),
                             dtype=torch.uint8, device=dev)

            def f8(cw, sw, x=x, y32=y32, y16=y16, ws=ws):
                return lambda: sg.skinny_gemm_fp8(x, cw, sw, y_f32=y32, y_bf16=y16, workspace=ws)
            nbytes = N * K + scales.numel() * 4 + M * K * 2 + M * N * 6
            run(label, M, N, K, lowp_plan_label("fp8", M, N, 0),
                [f8(cw, sw) for cw, sw in ring], nbytes)
        del ring
    # router scores + top-8 (E = 384, K = 7168)
    E, K, k = 384, 7168, 8
    W0 = si.normal_bf16((E, K), 0.02, 19, dev)
    ring = [W0] + [W0.clone() for _ in range(reps - 1)]
    for T in (1, 64):
        x = si.normal_bf16((T, K), 1.0, 20, dev)
        p = sg.skinny_gemm_plan(T, E, K)
        scores = torch.empty((T, E), device=dev)
        ws = torch.empty(max(p.workspace_bytes, 256), dtype=torch.uint8, device=dev)

        def rt(w, x=x, p=p, scores=scores, ws=ws):
            def go():
                L.projection(p, x, w, scores, None, ws)()
                sg.skinny_gemm_router_topk(scores, k)
            return go
        run("router top-8 E=384 K=7168", T, E, K, f"{desc(p)}+router_topk",
            [rt(w) for w in ring], proj_bytes(T, E, K, bf16=False) + T * E * 4 + T * k * 4)
    del ring, W0
    torch.cuda.empty_cache()
    with open(manifest_path, "w") as f:
        json.dump(manifest, f, indent=1)
    log(f"manifest: {manifest_path}")


def _dispatch_counters(directory: str):
    """Per dispatch of this library's kernels, in launch order: (kernel, {counter: value});
    and the calibration copy's counters."""
    rows = []
    for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            rows += list(csv.DictReader(f))
    if not rows:
        raise SystemExit(f"no counter_collection.csv under {directory}")
    disp = {}
    for r in rows:
        d = disp.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"],
                                                   "grid": int(r["Grid_Size"]), "c": {}})
        d["c"][r["Counter_Name"]] = d["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    ours = [disp[k] for k in sorted(disp) if "sg::" in disp[k]["name"]]
    calib = [d["c"] for d in disp.values()
             if COPY_KERNEL_TAG in d["name"] and d["grid"] == COPY_GRID]
    return ours, calib


def summarize_workloads(manifest_path: str, dirs) -> None:
    """Per workload and kernel: HBM bytes (FETCH_SIZE + WRITE_SIZE, each scaled by the
    calibration copy), their ratio to the algorithmic bytes, and the utilisation
    counters, from rocprofv3 --pmc passes over `bench.py --profile-workloads`."""
    with open(manifest_path) as f:
        manifest = json.load(f)
    per = {}  # (workload index, kernel short name) -> {counter: [values]}
    scale = {}
    for d in dirs:
        ours, calib = _dispatch_counters(d)
        for c in calib:
            for name in ("FETCH_SIZE", "WRITE_SIZE"):
                if name in c:
                    scale[name] = c[name] * 1024 / COPY_BYTES
        need = sum(w["dispatches"] for w in manifest)
        if len(ours) != need:
            raise SystemExit(f"{d}: {len(ours)} dispatches of the library, manifest expects {need}")
        i = 0
        for wi, w in enumerate(manifest):
            for _ in range(w["dispatches"]):
                k = ours[i]
                i += 1
                short = k["name"].replace("void ", "").replace("sg::(anonymous namespace)::", "")
                short = short.split("(")[0]
                slot = per.setdefault((wi, short), {})
                for cname, v in k["c"].items():
                    slot.setdefault(cname, []).append(v)
    print("# Per-workload counters of this library's kernels (rocprofv3 --pmc, one pass each)")
    print("# commands (repository root; OUT = an output folder):")
    print("#   rocprofv3 --pmc FETCH_SIZE -f csv -d OUT/wl_fetch -o f -- python bench.py "
          "--profile-workloads OUT/wl_fetch.json")
    print("#   rocprofv3 --pmc WRITE_SIZE -f csv -d OUT/wl_write -o w -- python bench.py "
          "--profile-workloads OUT/wl_write.json")
    print("#   rocprofv3 --pmc MfmaUtil LdsUtil VALUBusy -f csv -d OUT/wl_util -o u -- python "
          "bench.py --profile-workloads OUT/wl_util.json")
    print("#   python bench.py --summarize-workloads OUT/wl_fetch.json OUT/wl_fetch OUT/wl_write "
          "OUT/wl_util")
    print(f"# HBM bytes = FETCH_SIZE / {scale.get('FETCH_SIZE', float('nan')):.4f} + "
          f"WRITE_SIZE / {scale.get('WRITE_SIZE', float('nan')):.4f} (KiB -> bytes; factors from "
          f"a 1 GiB element-wise copy); per call = summed over the kernels of one call")
    print(f"# {'workload':34s} {'M':>3} {'kernel':44s} {'HBM MB':>8} {'x alg':>6} "
          f"{'Mfma%':>6} {'Lds%':>6} {'VALU%':>6}")
    for wi, w in enumerate(manifest):
        for (wj, short), c in per.items():
            if wj != wi:
                continue
            mean = {k: sum(v) / len(v) for k, v in c.items()}
            hbm = None
            if "FETCH_SIZE" in mean and "WRITE_SIZE" in mean and scale:
                hbm = (mean["FETCH_SIZE"] * 1024 / scale["FETCH_SIZE"] +
                       mean["WRITE_SIZE"] * 1024 / scale["WRITE_SIZE"])
            ratio = hbm / w["bytes_per_call"] if hbm is not None else float("nan")

            def pct(k):
                return f"{mean[k]:6.1f}" if k in mean else f"{'-':>6}"
            print(f"  {w['workload'][:34]:34s} {w['M']:3d} {short[:44]:44s} "
                  f"{(hbm or float('nan')) / 1e6:8.2f} {ratio:6.3f} "
                  f"{pct('MfmaUtil')} {pct('LdsUtil')} {pct('VALUBusy')}")
        print(f"  {'':34s} {'':3s} {'  algorithmic bytes per call':44s} "
              f"{w['bytes_per_call'] / 1e6:8.2f}   plan: {w['plan']}")


def copy_calibration(torch, nbytes=COPY_BYTES, reps=3):
    """A plain element-wise copy of known size (reads nbytes, writes nbytes) for scaling
    the FETCH_SIZE / WRITE_SIZE counters."""
    src = torch.ones(nbytes // 4, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    log(f"copy calibration: {reps} element-wise copies of {nbytes} bytes")


# --------------------------------------------------------------------------- main


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--jsonl", metavar="PATH",
                    help="write the sweep's rows to PATH as JSON lines, section by section; "
                         "run again with the same PATH to resume a killed sweep")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-trace", nargs=2, metavar=("DIR", "COMMAND"))
    ap.add_argument("--profile-workloads", metavar="MANIFEST")
    ap.add_argument("--side-stream-cu-mask", type=int, metavar="CUS",
                    help="time the MoE step with the shared expert on a stream masked to the "
                         "first CUS compute units, then exit")
    ap.add_argument("--summarize-workloads", nargs="+", metavar="MANIFEST_THEN_DIRS")
    args = ap.parse_args()

    if args.summarize_workloads:
        summarize_workloads(args.summarize_workloads[0], args.summarize_workloads[1:])
        return

    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(collectives are out of scope), so --gpus must be 1", file=sys.stderr)
        raise SystemExit(2)

    import torch

    import seeded_inputs as si
    import skinny_gemm_projection_amd as sg

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs an MI355X (no GPU visible)")
    torch.cuda.set_device(0)
    L = Launcher(torch, sg)
    cyc = sleep_cycles_per_ms(torch)
    if args.profile_workloads:
        profile_workloads(torch, sg, si, L, args.profile_workloads)
        return
    if args.side_stream_cu_mask:
        if not 1 <= args.side_stream_cu_mask <= 256:
            raise SystemExit("--side-stream-cu-mask: 1..256 compute units")
        rows = side_stream_cu_mask(torch, sg, si, L, cyc, args.side_stream_cu_mask)
        print(json.dumps({"experiment": "MoE step, shared expert on a CU-masked side stream",
                          "rows": rows}), flush=True)
        return
    if args.copy_calibration:
        copy_calibration(torch)

    log(f"main workload: M in {M_LIST}, K={K_MAIN}, N={N_MAIN}, steps={args.steps}, "
        f"warmup={args.warmup}")
    res = main_workload(torch, sg, si, L, args.steps, args.warmup, cyc)
    log(f"value {res['value']:.1f} GB/s, {res['ms_per_step'] * 1e3:.2f} us/step, "
        f"per projection {res['us_per_projection']}")

    sweep_rows = None
    if not args.no_sweep:
        log("sweep over batch sizes and workloads")
        sweep_rows = sweep(torch, sg, si, L, cyc,
                           journal=SweepJournal(args.jsonl) if args.jsonl else None)
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline: the fp64 oracle on this host")
        cpu = cpu_baseline(si, res["inputs"])

    traffic = read_traffic()
    line = {
        "metric": "µs/projection and achieved HBM GB/s (% of peak) vs batch M=1..64",
        "value": round(res["value"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "accumulate": "fp32",
        "data": "synthetic",
        "config": {
            "workload": "small-batch decode projection y = x W^T, M in {1,2}, K=7168, N=8192, "
                        "bf16 x~N(0,1), W~N(0,0.02^2), fp32+bf16 outputs; one step = the M=1 "
                        "and the M=2 call",
            "M": list(M_LIST), "N": N_MAIN, "K": K_MAIN,
            "weight_ring_copies": res["ring_copies"], "weight_ring_bytes": res["ring_bytes"],
            "parallelism": "single GPU",
        },
        "us_per_projection": res["us_per_projection"],
        "us_per_projection_graph": res["graph"],
        "us_single_call_cold": res["cold"],
        "GBps_per_batch": res["gbs_per_batch"],
        "pct_of_peak": round(100.0 * res["value"] / HBM_PEAK_GBS, 1),
        "wall_ms_per_step": round(res["wall_ms_per_step"], 6),
        "roofline": {
            "bound": "hbm",
            "kernel": "rowstream_kernel (small-matrix path, M=1 and M=2)",
            "achieved": round(res["achieved"], 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(res["achieved"] / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "bytes_per_launch": round(res["bytes_per_launch"]),
            "avg_launch_us": round(res["avg_launch_us"], 3),
            # the same launches with the arithmetic, reduction and stores taken out (the
            # library's read probe): the read rate this kernel's load shape reaches here
            "read_probe": res["read_probe"],
        },
        "cpu_baseline": cpu,
    }
    if sweep_rows is not None:
        line["sweep"] = sweep_rows
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

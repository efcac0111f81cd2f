#!/usr/bin/env python3
"""Throughput of the MoE dispatch / combine hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config prefill]

One step = the whole forward hot path over one batch of the workload:
dispatch layout -> FP8 dispatch (pack + quantize) -> combine (weighted
gather-reduce to bf16), all inputs resident in HBM. By default the layout
and the dispatch are one launch (ep_dispatch_with_layout) and steps are
captured in a HIP graph (up to 10 per graph) and replayed to run exactly K
(--eager: plain launches; --separate: three calls). `value` is dispatch + combine algorithmic bytes per
second of step time (GB/s); the JSON line also carries the eager step, the
per-kernel breakdown (events around eager launches), the roofline of the
dominant kernel, the decode latency at 128 tokens, the backward pair, the
skewed and large workloads' steps (`other_workloads`), and the CPU oracle
baseline.
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

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", default="prefill")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extras", action="store_true", help="skip decode/backward/copy extras")
    p.add_argument("--no-decode", action="store_true", help="skip the decode-latency extra")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--eager", action="store_true",
                   help="time the step as eager launches instead of replays of a HIP graph holding one step")
    p.add_argument("--separate", action="store_true",
                   help="time the step as three calls (layout, dispatch, combine) instead of the fused "
                        "layout+dispatch launch followed by combine")
    p.add_argument("--tokens-per-rank", action="store_true",
                   help="read the workload's token count as per source rank (T x R tokens on the GPU) "
                        "instead of per GPU")
    p.add_argument("--ll", action="store_true",
                   help="time the low-latency form as the step (one dispatch launch into fixed "
                        "per-(expert, source) regions, then combine); implies --no-extras")
    p.add_argument("--dedup", action="store_true",
                   help="time the rank-deduplicated form as the step (layout, one row per (token, rank), "
                        "combine of the pre-reduced rows); implies --no-extras")
    p.add_argument("--record-counters", nargs="+", metavar="PASS_DIR",
                   help="summarize rocprofv3 --pmc runs of this bench (one counter set per run, "
                        "--output-format csv; the sets of COUNTER_PASSES) into profiles/")
    p.add_argument("--patterns-only", action="store_true",
                   help="after the timed steps, run only the access-pattern leg and print its figures "
                        "(a short run for a kernel trace of the pattern kernels)")
    p.add_argument("--record-patterns", metavar="TRACE_DIR",
                   help="summarize a rocprofv3 --kernel-trace --stats run of this bench with --patterns-only "
                        "(--output-format csv) into profiles/")
    p.add_argument("--record-traffic", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "TRACE_DIR"),
                   help="summarize rocprofv3 runs of this bench (--pmc FETCH_SIZE, --pmc WRITE_SIZE, "
                        "--kernel-trace --stats, all with --output-format csv) into profiles/")
    return p.parse_args()


def algo_bytes(T, k, H, N, use_fp8):
    """Bytes the method must move (kept slots N): reads of x and weights and
    positions, writes of the rows, scales and received weights; combine reads
    the rows and writes y."""
    G = H // 128
    if use_fp8:
        d = 2 * T * H + N * H + 4 * N * G + 4 * N + 8 * T * k
    else:
        d = 2 * T * H + 2 * N * H + 4 * N + 8 * T * k
    c = 2 * N * H + 2 * T * H + 8 * T * k
    cb = 2 * T * H + 2 * N * H + 4 * T * k
    return d, c, cb


class Path:
    """Device buffers and the step of one workload (everything preallocated)."""

    def __init__(self, cfg, seed, torch, ep, workloads):
        self.cfg = cfg
        self.torch = torch
        wl = workloads.make_workload(cfg, seed=seed)
        self.wl = wl
        dev = "cuda"
        self.x = torch.from_numpy(wl.x.view("int16")).to(dev).view(torch.bfloat16)
        self.topk = torch.from_numpy(wl.topk_idx).to(dev)
        self.w = torch.from_numpy(wl.topk_w).to(dev)
        # receive capacity: the largest per-rank row count (one layout on a
        # provisional context, outside any timing)
        probe = ep.Buffer(cfg.T, cfg.H, cfg.k, cfg.E, cfg.R, cfg.T * cfg.k)
        Lp = probe.get_dispatch_layout(self.topk)
        self.cap = int(Lp.rank_rows.max().item()) if cfg.T else 0
        probe.status()
        probe.close()
        self.buf = ep.Buffer(cfg.T, cfg.H, cfg.k, cfg.E, cfg.R, self.cap)
        b = self.buf
        self.layout = b.new_layout()
        n = b.num_rows
        self.recv_x = torch.empty((n, cfg.H), dtype=torch.uint8 if cfg.use_fp8 else torch.bfloat16, device=dev)
        self.recv_scales = torch.empty((n, cfg.H // 128), dtype=torch.float32, device=dev) if cfg.use_fp8 else None
        self.recv_w = torch.empty(n, dtype=torch.float32, device=dev)
        self.handle = b.new_handle()
        self.expert_out = workloads.device_normal_bf16((n, cfg.H), seed=seed + 101)
        self.y = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device=dev)
        self.grad_y = None

    def layout_op(self):
        self.buf.get_dispatch_layout(self.topk, self.layout)

    def dispatch_op(self):
        self.buf.dispatch(self.x, self.topk, self.w, self.layout, self.cfg.use_fp8,
                          out=(self.recv_x, self.recv_scales, self.recv_w, self.handle))

    def fused_op(self):
        self.buf.dispatch_with_layout(self.x, self.topk, self.w, self.cfg.use_fp8, layout=self.layout,
                                      out=(self.recv_x, self.recv_scales, self.recv_w, self.handle))

    def combine_op(self):
        self.buf.combine(self.expert_out, self.handle, self.w, out=self.y)

    def kept_slots(self):
        return int((self.handle.pos >= 0).sum().item())


class LlPath:
    """The low-latency form of a workload's step: one dispatch launch into
    fixed per-(expert, source) regions, then combine on its handle."""

    def __init__(self, main, torch, ep, workloads, seed, init_rows=True):
        cfg = main.cfg
        self.main = main
        self.buf = ep.Buffer(cfg.T, cfg.H, cfg.k, cfg.E, cfg.R, ep.ll_cap_rows(cfg.T, cfg.E, cfg.R))
        n = self.buf.num_rows
        self.recv_x = torch.empty((n, cfg.H), dtype=torch.uint8 if cfg.use_fp8 else torch.bfloat16, device="cuda")
        self.recv_scales = torch.empty((n, cfg.H // 128), dtype=torch.float32, device="cuda") if cfg.use_fp8 else None
        self.recv_w = torch.empty(n, dtype=torch.float32, device="cuda")
        self.recv_count = torch.empty((cfg.E, cfg.R), dtype=torch.int32, device="cuda")
        self.handle = self.buf.new_handle()
        # expert outputs for every receive row (E*T of them; timing-only
        # copies may leave them uninitialized: the values do not change the work)
        self.expert_out = (workloads.device_normal_bf16((n, cfg.H), seed=seed + 404) if init_rows
                           else torch.empty((n, cfg.H), dtype=torch.bfloat16, device="cuda"))
        self.y = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device="cuda")

    def dispatch_op(self):
        m = self.main
        self.buf.dispatch_low_latency(m.x, m.topk, m.w, m.cfg.use_fp8,
                                      out=(self.recv_x, self.recv_scales, self.recv_w, self.recv_count,
                                           self.handle))

    def combine_op(self):
        self.buf.combine(self.expert_out, self.handle, self.main.w, out=self.y)


def dedup_bytes(T, k, H, Nd, N, use_fp8):
    """Algorithmic bytes of the rank-deduplicated step (Nd = rows, one per
    (token, destination rank); N = kept (token, expert) slots): dispatch
    reads x and the weights, writes the rows (+ scales) and each row's k
    routing entries (index + weight); the expert-side pre-reduction reads the
    N expert outputs of the rows' kept slots and the rows' routing entries
    and writes the Nd reduced rows; the combine of the reduced rows reads them
    and writes y. Returns (dispatch, pre-reduction, combine)."""
    G = H // 128
    row = H + 4 * G if use_fp8 else 2 * H
    d = 2 * T * H + Nd * row + 8 * Nd * k + 4 * T * k
    pre = 2 * N * H + 8 * Nd * k + 2 * Nd * H
    c = 2 * Nd * H + 2 * T * H + 4 * T * k
    return d, pre, c


class DedupPath:
    """The rank-deduplicated form of a workload's step: layout with the
    leader ranks, one row per (token, destination rank), the expert-side
    pre-reduction of each row's expert outputs (per (row, slot), N(0,1)
    bf16), and the combine of the reduced rows (unit weights)."""

    def __init__(self, main, torch, ep, workloads, seed):
        cfg = main.cfg
        self.main = main
        probe = ep.Buffer(cfg.T, cfg.H, cfg.k, cfg.E, cfg.R, cfg.T)
        Lp = probe.get_dispatch_layout(main.topk, probe.new_layout(dedup=True))
        self.cap = int(Lp.token_rows.max().item()) if cfg.T else 0
        probe.status()
        probe.close()
        self.buf = ep.Buffer(cfg.T, cfg.H, cfg.k, cfg.E, cfg.R, self.cap)
        b = self.buf
        n = b.num_rows
        self.layout = b.new_layout(dedup=True)
        self.recv_x = torch.empty((n, cfg.H), dtype=torch.uint8 if cfg.use_fp8 else torch.bfloat16, device="cuda")
        self.recv_scales = torch.empty((n, cfg.H // 128), dtype=torch.float32, device="cuda") if cfg.use_fp8 else None
        self.recv_topk_idx = torch.empty((n, cfg.k), dtype=torch.int32, device="cuda")
        self.recv_topk_w = torch.empty((n, cfg.k), dtype=torch.float32, device="cuda")
        self.handle = b.new_handle()
        self.expert_out = workloads.device_normal_bf16((n, cfg.k, cfg.H), seed=seed + 303)
        self.reduced = torch.empty((n, cfg.H), dtype=torch.bfloat16, device="cuda")
        self.y = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device="cuda")

    def layout_op(self):
        self.buf.get_dispatch_layout(self.main.topk, self.layout)

    def dispatch_op(self):
        m = self.main
        self.buf.dispatch_dedup(m.x, m.topk, m.w, self.layout, m.cfg.use_fp8,
                                out=(self.recv_x, self.recv_scales, self.recv_topk_idx, self.recv_topk_w,
                                     self.handle))

    def fused_op(self):
        m = self.main
        self.buf.dispatch_dedup_with_layout(m.x, m.topk, m.w, m.cfg.use_fp8, layout=self.layout,
                                            out=(self.recv_x, self.recv_scales, self.recv_topk_idx,
                                                 self.recv_topk_w, self.handle))

    def prereduce_op(self):
        self.buf.prereduce(self.expert_out, self.recv_topk_idx, self.recv_topk_w, self.layout.token_rows,
                           out=self.reduced)

    def combine_op(self):
        self.buf.combine(self.reduced, self.handle, None, out=self.y)

    def rows(self):
        return int((self.handle.pos >= 0).sum().item())


def stream_timed(torch, stream, ops, K, W):
    """ops launched K times back to back on one stream (after W), timed by
    events on that stream: no cross-queue waits inside the timed region."""
    with torch.cuda.stream(stream):
        for _ in range(W):
            for op in ops:
                op()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(K):
            for op in ops:
                op()
        e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) / K


def concurrent_timed(torch, streams_ops, K, W):
    """Each (stream, ops) pair launched on its own stream at once, the host
    synchronizing between repetitions; a repetition lasts from the earliest
    start event to the latest end event (one device clock for all streams).
    Returns the mean over K repetitions (after W)."""
    reps = []
    for i in range(W + K):
        torch.cuda.synchronize()
        marks = []
        for st, ops in streams_ops:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(st)
            with torch.cuda.stream(st):
                for op in ops:
                    op()
            e1.record(st)
            marks.append((e0, e1))
        if i >= W:
            reps.append(marks)
    torch.cuda.synchronize()
    total = 0.0
    for marks in reps:
        ref = marks[0][0]
        starts = [ref.elapsed_time(a) for a, _ in marks]
        ends = [ref.elapsed_time(b) for _, b in marks]
        total += max(ends) - min(starts)
    return total / K


def units_used(torch, ep, stream):
    """Distinct compute units a census launch on `stream` ran on."""
    with torch.cuda.stream(stream):
        ids = ep.cu_census(8192)
    stream.synchronize()
    return int(torch.unique(ids).numel())


def cu_cap_overlap(torch, ep, p, K, W):
    """The exchange step (fused layout+dispatch, combine) on a stream held to
    n compute units while a bf16 GEMM runs on the other units: time of each
    alone and of both at once."""
    M, Kd, Nn = 4096, 7168, 4096
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    a = torch.randn((M, Kd), generator=g, device="cuda").to(torch.bfloat16)
    b = torch.randn((Kd, Nn), generator=g, device="cuda").to(torch.bfloat16).contiguous()
    c = torch.empty((M, Nn), dtype=torch.bfloat16, device="cuda")

    def gemm():
        torch.matmul(a, b, out=c)

    ep_ops = [p.fused_op, p.combine_op]
    full, other = torch.cuda.Stream(), torch.cuda.Stream()
    gemm_full = stream_timed(torch, full, [gemm], K, W)
    ep_full = stream_timed(torch, full, ep_ops, K, W)
    both_full = concurrent_timed(torch, [(full, ep_ops), (other, [gemm])], K, W)
    flops = 2.0 * M * Kd * Nn
    res = {"gemm": {"shape_mkn": [M, Kd, Nn], "dtype": "bf16", "us": round(gemm_full * 1e3, 2),
                    "TFLOPs": round(flops / (gemm_full * 1e-3) / 1e12, 1)},
           "exchange_us": round(ep_full * 1e3, 2),
           "serial_us": round((gemm_full + ep_full) * 1e3, 2),
           "by_cus": {"256 (shared, no cap)": {"both_us": round(both_full * 1e3, 2)}}}
    for n in (32, 64, 128, 192):
        p.buf.set_num_cus(n)
        with ep.CuStream(n) as cs, ep.CuStream(n, exclude=True) as rest:
            units = [units_used(torch, ep, st) for st in (cs.torch_stream, rest.torch_stream)]
            e_ms = stream_timed(torch, cs.torch_stream, ep_ops, K, W)
            g_ms = stream_timed(torch, rest.torch_stream, [gemm], K, W)
            b_ms = concurrent_timed(torch, [(cs.torch_stream, ep_ops), (rest.torch_stream, [gemm])], K, W)
        p.buf.set_num_cus(0)
        res["by_cus"][str(n)] = {"units_seen": units, "exchange_alone_us": round(e_ms * 1e3, 2),
                                 "gemm_on_other_units_us": round(g_ms * 1e3, 2),
                                 "both_us": round(b_ms * 1e3, 2)}
    if p.buf.status():
        raise SystemExit(f"bench: device status {p.buf.status()} in the overlap runs")
    del a, b, c
    return res


def timed(torch, ops, K, W, stats=None):
    """W untimed warmups, then exactly K steps between synchronizations; HIP
    events (torch's current stream = the launch stream) bracket every op
    (their p10 / median / p90 go to `stats` when given)."""
    for _ in range(W):
        for op in ops:
            op()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(ops) + 1)] for _ in range(K)]
    t0 = time.perf_counter()
    for i in range(K):
        ev[i][0].record()
        for j, op in enumerate(ops):
            op()
            ev[i][j + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_op = [sum(ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(K)) / K for j in range(len(ops))]
    if stats is not None:  # p10 / median / p90 of every op, in ms
        for j in range(len(ops)):
            xs = sorted(ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(K))
            stats.append(tuple(xs[min(K - 1, int(q * K))] for q in (0.1, 0.5, 0.9)))
    return wall / K * 1e3, per_op  # ms per step, ms per op


def back_to_back_rotating(torch, ops, K, W):
    """K launches of one op, cycling through the sets' copies of it (`ops`),
    back to back between two HIP events on the launch stream: the per-launch
    duration with no event between launches and no set's data left in the
    memory-side cache by the launch before. Returns ms per launch."""
    n = len(ops)
    for i in range(W):
        ops[i % n]()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(K):
        ops[i % n]()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / K


def timed_rotating(torch, sets_ops, K, W, stats=None):
    """timed() over steps that cycle through the sets (step i runs
    sets_ops[i % n]); each op kind's event times are pooled over the sets."""
    n = len(sets_ops)
    for i in range(W):
        for op in sets_ops[i % n]:
            op()
    torch.cuda.synchronize()
    m = len(sets_ops[0])
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(m + 1)] for _ in range(K)]
    t0 = time.perf_counter()
    for i in range(K):
        ev[i][0].record()
        for j, op in enumerate(sets_ops[i % n]):
            op()
            ev[i][j + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_op = [sum(ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(K)) / K for j in range(m)]
    if stats is not None:
        for j in range(m):
            xs = sorted(ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(K))
            stats.append(tuple(xs[min(K - 1, int(q * K))] for q in (0.1, 0.5, 0.9)))
    return wall / K * 1e3, per_op


def graph_rotating(torch, sets_ops, K, W):
    """K steps cycling through the sets, captured in HIP graphs of G steps
    (G = the largest divisor of K up to 200) and replayed K / G times after
    untimed replays covering W steps. Returns (ms per step by wall clock, ms
    per step by events, G)."""
    n = len(sets_ops)
    G = max(d for d in range(1, min(K, 200) + 1) if K % d == 0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for ops in sets_ops:  # first calls outside the capture
            for op in ops:
                op()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(G):
            for op in sets_ops[i % n]:
                op()
    for _ in range((W + G - 1) // G):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(K // G):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall / K * 1e3, e0.elapsed_time(e1) / K, G


def graph_step_timed(torch, ops, K, W):
    """G consecutive steps captured in one HIP graph (G = the largest divisor
    of K up to 10, as a forward pass captures its layers together); untimed
    replays for the W warmup steps, then exactly K steps (K / G replays)
    between synchronizations. Returns (ms per step by wall clock, ms per step
    by events on the replay stream, G)."""
    G = max(d for d in range(1, 11) if K % d == 0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for op in ops:  # first calls (library load, allocations) outside the capture
            op()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(G):
            for op in ops:
                op()
    for _ in range((W + G - 1) // G):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(K // G):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall / K * 1e3, e0.elapsed_time(e1) / K, G


def graph_timed(torch, ops, K, W, inner=20):
    """Capture `inner` consecutive steps in one HIP graph (the launch-bound
    decode path), replay it; returns (GPU us per step from events, wall us per
    step). Capture follows a warmup on a side stream, as torch requires."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(W):
            for op in ops:
                op()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(inner):
            for op in ops:
                op()
    g.replay()
    torch.cuda.synchronize()
    reps = max(1, K // inner)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    n = reps * inner
    return e0.elapsed_time(e1) * 1e3 / n, wall * 1e6 / n


def pattern_floors(torch, ep, steps, sets, K, W, d_bytes, c_bytes, N):
    """The step's memory-access patterns with none of its arithmetic (the
    ep_pattern_* utilities), each timed like the dominant kernel (K launches
    back to back over the rotated sets), beside the fused launch and the
    combine timed the same way: the rate the HBM sustains for the pattern a
    kernel must make, against which its own rate is compared.
      push    x row read, then k scattered FP8-sized row writes per token
      gather  k scattered row reads, then one row write per token (at the
              combine's residency cap, and uncapped)
      fill    compact writes of the dispatch's row bytes
      read    compact reads of the combine's row bytes"""
    cfg = sets[0].cfg
    T, k, H = cfg.T, cfg.k, cfg.H
    nrows = sets[0].buf.num_rows
    strm = lambda: torch.cuda.current_stream().cuda_stream
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    ms = lambda ops: back_to_back_rotating(torch, ops, K, W)
    out = {"timing": f"{K} launches back to back between two HIP events, cycling through the {len(sets)} "
                     "rotated sets (as the dominant kernel)"}
    fused_ms = ms([st[0][0] for st in steps])
    comb_ms = ms([st[0][-1] for st in steps])
    gath_ms = ms([lambda q=q: ep.ep_pattern_gather(q.expert_out.data_ptr(), q.handle.pos.data_ptr(), q.y.data_ptr(),
                                                   T, k, H, nrows, True, strm()) for q in sets])
    gath_u_ms = ms([lambda q=q: ep.ep_pattern_gather(q.expert_out.data_ptr(), q.handle.pos.data_ptr(),
                                                     q.y.data_ptr(), T, k, H, nrows, False, strm()) for q in sets])
    r_bytes = (2 * N * H) // 4096 * 4096
    read_ms = ms([lambda q=q: ep.ep_pattern_read(q.expert_out.data_ptr(), r_bytes, sink.data_ptr(), strm())
                  for q in sets])
    g_bytes = 2 * N * H + 2 * T * H
    out["combine"] = {"us": round(comb_ms * 1e3, 2), "GBps": round(c_bytes / (comb_ms * 1e-3) / 1e9, 1)}
    out["gather_capped"] = {"us": round(gath_ms * 1e3, 2), "bytes": g_bytes,
                            "GBps": round(g_bytes / (gath_ms * 1e-3) / 1e9, 1)}
    out["gather_uncapped"] = {"us": round(gath_u_ms * 1e3, 2), "GBps": round(g_bytes / (gath_u_ms * 1e-3) / 1e9, 1)}
    out["read_compact"] = {"bytes": r_bytes, "GBps": round(r_bytes / (read_ms * 1e-3) / 1e9, 1)}
    out["combine_rate_over_gather"] = round((c_bytes / comb_ms) / (g_bytes / gath_ms), 4)
    out["layout_dispatch"] = {"us": round(fused_ms * 1e3, 2), "GBps": round(d_bytes / (fused_ms * 1e-3) / 1e9, 1)}
    if cfg.use_fp8 and H <= 8192:
        push_ms = ms([lambda q=q: ep.ep_pattern_push(q.x.data_ptr(), q.handle.pos.data_ptr(), q.recv_x.data_ptr(),
                                                     T, k, H, nrows, strm()) for q in sets])
        p_bytes = 2 * T * H + N * H
        w_bytes = min(N * (H + H // 32), sets[0].recv_x.numel() * sets[0].recv_x.element_size()) // 1024 * 1024
        fill_ms = ms([lambda q=q: ep.ep_pattern_fill(q.recv_x.data_ptr(), w_bytes, strm()) for q in sets])
        out["push"] = {"us": round(push_ms * 1e3, 2), "bytes": p_bytes,
                       "GBps": round(p_bytes / (push_ms * 1e-3) / 1e9, 1)}
        out["fill_compact"] = {"bytes": w_bytes, "GBps": round(w_bytes / (fill_ms * 1e-3) / 1e9, 1)}
        out["layout_dispatch_rate_over_push"] = round((d_bytes / fused_ms) / (p_bytes / push_ms), 4)
        step_floor = d_bytes / (p_bytes / push_ms) + c_bytes / (g_bytes / gath_ms)
        out["step_at_pattern_rates_us"] = round(step_floor * 1e3, 2)
    return out


def source_sha():
    h = hashlib.sha256()
    for f in ("ep_kernels.hip", "ep_api.hip", "ep_internal.h"):
        with open(os.path.join(ROOT, "combine_get_dispatch_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch (calibrated FETCH_SIZE + WRITE_SIZE) from the
    committed rocprofv3 counter summary, if it was taken on the current
    kernel sources (else None)."""
    path = os.path.join(PROFILES, "traffic.json")
    try:
        with open(path) as f:
            d = json.load(f)[workload]
        if d.get("source_sha") != source_sha():
            return None
        return d[kernel]["hbm_bytes_per_launch"]
    except (OSError, KeyError, ValueError):
        return None


# ---------------------------------------------------------------------------
# rocprofv3 summaries -> profiles/
# ---------------------------------------------------------------------------

KERNELS = {  # regular expressions on the kernel names rocprofv3 reports
    "k_layout": r"k_layout<", "k_layout_dispatch": r"k_layout_dispatch<\d+, \w+, 1>",
    "k_layout_dispatch_dedup": r"k_layout_dispatch<\d+, \w+, 2>", "k_dispatch": r"k_dispatch<true, 1(, \w+)?>",
    "k_dispatch_dedup": r"k_dispatch<true, 2(, \w+)?>", "k_ll_dispatch": r"k_ll_dispatch<",
    "k_combine": r"k_combine<false,", "k_prereduce": r"k_prereduce<false", "k_copy": r"k_copy"}


def _csv_rows(d, suffix):
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)
    if not files:
        raise SystemExit(f"no *{suffix} under {d}")
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def _per_kernel(rows, value_key):
    """Dispatches per kernel of interest in launch order (the bench runs the
    warmup and timed steps of the main loop first, so the first instances of
    k_combine<false, *> are the forward combine, not dispatch_backward)."""
    out = {k: [] for k in KERNELS}
    for r in sorted(rows, key=lambda r: int(r.get("Dispatch_Id", r.get("Correlation_Id", 0)))):
        for k, pat in KERNELS.items():
            if re.search(pat, r["Kernel_Name"]):
                out[k].append((int(r["Grid_Size"]), float(r[value_key])))
    return out


# One rocprofv3 --pmc run per set (a run holds at most 4 TCC and 8 SQ counters).
COUNTER_PASSES = [
    "MeanOccupancyPerCU MeanOccupancyPerActiveCU OccupancyPercent",
    "TCC_EA0_RDREQ_sum TCC_EA0_RDREQ_LEVEL_sum TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum TCC_TAG_STALL_sum",
    "TCC_EA0_WRREQ_sum TCC_EA0_WRREQ_LEVEL_sum TCC_EA0_WRREQ_DRAM_CREDIT_STALL_sum TCC_EA0_WRREQ_STALL_sum",
    "TCC_EA0_WRREQ_64B_sum TCC_TOO_MANY_EA_WRREQS_STALL_sum TCC_EA0_RDREQ_128B_sum TCC_EA0_RDREQ_64B_sum",
]
# waves per SIMD the code objects allow (VGPRs; for the combine of a long
# launch, the LDS each two-wave workgroup reserves: 4 per CU), for the
# occupancy bound (compiler resource-usage remarks of this build: k_layout<8>
# and the top-8 fused grids 113 VGPRs, the FP8 per-expert dispatch 91, the
# per-rank one 99, the combine 92, the four-row pre-reduction 143, the
# one-pass top-8 FP8 low-latency dispatch 56, the copy 10)
COMBINE_CAP_MIN_WAVES = 64 * 256  # the combine runs capped from 64 waves per CU (256 CUs)
WAVES_PER_SIMD_BOUND = {"k_layout": 4, "k_layout_dispatch": 4, "k_layout_dispatch_dedup": 4, "k_dispatch": 5,
                        "k_dispatch_dedup": 4, "k_ll_dispatch": 8, "k_combine": 2, "k_prereduce": 3, "k_copy": 8}


def record_counters(args, cfg):
    """Per-kernel means of the counters in the given rocprofv3 --pmc output
    directories, and what they imply: occupancy against the code objects'
    bound, mean L2-to-memory read and write latency, DRAM credit stall
    cycles per request, request sizes. Writes profiles/<workload>_counters.md."""
    vals = {}
    passes = []
    for d in args.record_counters:
        rows = _csv_rows(d, "counter_collection.csv")
        names = sorted({r["Counter_Name"] for r in rows})
        passes.append(" ".join(names))
        for k, pat in KERNELS.items():
            for r in rows:
                if re.search(pat, r["Kernel_Name"]):
                    vals.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    mean = lambda xs: sum(xs) / len(xs)
    cmd = (f"python3 bench.py --config {cfg.name}{mode_flags(args)} --steps {args.steps} --warmup {args.warmup} "
           "--no-cpu-baseline --no-decode --no-extras")
    lines = [f"# {cfg.name}{mode_flags(args).replace(' --', '_')}: occupancy and memory-request counters (rocprofv3)",
             "", f"Workload: {cfg.desc}.", "",
             "Commands (run from /tmp with TMPDIR=/tmp; the bench runs from the repository root), one run per "
             "counter set:", ""]
    for i, ps in enumerate(passes):
        lines.append(f"    rocprofv3 --pmc {ps} --output-format csv -d <pass{i + 1}> -o run -- {cmd}")
    lines += [f"    python3 bench.py --config {cfg.name}{mode_flags(args)} --steps {args.steps} --warmup {args.warmup} "
              "--record-counters " + " ".join(f"<pass{i + 1}>" for i in range(len(passes))), "",
              "Means over the profiled launches of each kernel. Occupancy: OccupancyPercent is the mean of "
              "resident waves over a CU's 32 wave slots (4 SIMDs x 8) while the kernel runs; the bound is what "
              "the code object's VGPR count allows (for the combine of a long launch, the LDS its two-wave "
              "workgroups reserve). Latencies are TCC (L2) cycles from a request leaving L2 to "
              "its return (LEVEL / REQ); credit stalls are cycles summed over the L2 channels.", "",
              "| kernel | launches | occupancy % | waves/CU | bound waves/CU | read latency | write latency | "
              "read credit stall / req | write credit stall / req | 128B reads % | 64B writes % |",
              "|---|---|---|---|---|---|---|---|---|---|---|"]
    for k, c in vals.items():
        g = lambda n: mean(c[n]) if n in c else None
        occ = g("OccupancyPercent")
        rd, rdl, rds = g("TCC_EA0_RDREQ_sum"), g("TCC_EA0_RDREQ_LEVEL_sum"), g("TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum")
        wr, wrl, wrs = g("TCC_EA0_WRREQ_sum"), g("TCC_EA0_WRREQ_LEVEL_sum"), g("TCC_EA0_WRREQ_DRAM_CREDIT_STALL_sum")
        r128, w64 = g("TCC_EA0_RDREQ_128B_sum"), g("TCC_EA0_WRREQ_64B_sum")
        f = lambda v, fmt: "-" if v is None else fmt.format(v)
        div = lambda a, b: None if a is None or not b else a / b
        nl = max(len(v) for v in c.values())
        bound = WAVES_PER_SIMD_BOUND.get(k)
        if k == "k_combine" and cfg.T * -(-cfg.H // 1024) < COMBINE_CAP_MIN_WAVES:
            bound = 5  # a short combine runs uncapped: its VGPRs (92) bound it
        lines.append(f"| `{k}` | {nl} | {f(occ, '{:.1f}')} | {f(None if occ is None else occ * 32 / 100, '{:.1f}')} | "
                     f"{f(None if bound is None else 4 * bound, '{:d}')} | {f(div(rdl, rd), '{:.0f}')} | "
                     f"{f(div(wrl, wr), '{:.0f}')} | {f(div(rds, rd), '{:.3f}')} | {f(div(wrs, wr), '{:.3f}')} | "
                     f"{f(None if div(r128, rd) is None else 100 * div(r128, rd), '{:.1f}')} | "
                     f"{f(None if div(w64, wr) is None else 100 * div(w64, wr), '{:.1f}')} |")
    lines += ["", "Raw means per kernel:", ""]
    for k, c in vals.items():
        lines.append(f"- `{k}`: " + ", ".join(f"{n} {mean(v):.4g}" for n, v in sorted(c.items())))
    lines += ["", f"Kernel sources: sha256 prefix {source_sha()} (ep_kernels.hip, ep_api.hip, ep_internal.h)."]
    path = os.path.join(PROFILES, f"{traffic_key(cfg, args)}_counters.md")
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    return path


def pattern_bytes(cfg, N):
    """Bytes each measured kernel of the access-pattern leg moves (as
    pattern_floors counts them): the step's two kernels' algorithmic bytes and
    the patterns' own."""
    T, k, H = cfg.T, cfg.k, cfg.H
    d, c, _ = algo_bytes(T, k, H, N, cfg.use_fp8)
    return {"k_layout_dispatch": d, "k_combine": c, "k_pattern_push": 2 * T * H + N * H,
            "k_pattern_gather": 2 * N * H + 2 * T * H, "k_pattern_fill": N * (H + H // 32) // 1024 * 1024,
            "k_pattern_read": (2 * N * H) // 4096 * 4096}


PATTERN_KERNELS = {  # rocprofv3 kernel names
    "k_layout_dispatch": r"k_layout_dispatch<\d+, \w+, 1>", "k_combine": r"k_combine<false, 2>",
    "k_pattern_push": r"k_pattern_push", "k_pattern_gather": r"k_pattern_gather<2>",
    "k_pattern_gather_uncapped": r"k_pattern_gather<4>", "k_pattern_fill": r"k_pattern_fill",
    "k_pattern_read": r"k_pattern_read", "k_copy": r"k_copy"}


def record_patterns(args, cfg):
    """Average durations (rocprofv3 --kernel-trace --stats) of the step's two
    kernels and of the access-pattern kernels, and the rates they imply.
    Writes profiles/<workload>_access_patterns.md."""
    from combine_get_dispatch_amd import workloads as wlmod
    wl = wlmod.make_workload(cfg, seed=args.seed, with_x=False)
    N = int((wl.topk_idx >= 0).sum())
    nb = pattern_bytes(cfg, N)
    nb["k_pattern_gather_uncapped"] = nb["k_pattern_gather"]
    stats = _csv_rows(args.record_patterns, "kernel_stats.csv")
    rows = {}
    for key, pat in PATTERN_KERNELS.items():
        for r in stats:
            if re.search(pat, r["Name"]):
                rows[key] = (int(r["Calls"]), float(r["AverageNs"]) / 1e3)
    cmd = f"python3 bench.py --config {cfg.name} --steps {args.steps} --warmup {args.warmup} --no-cpu-baseline " \
          "--no-decode --no-extras --patterns-only"
    lines = [f"# {cfg.name}: the step's kernels beside their access patterns (rocprofv3 kernel trace)", "",
             f"Workload: {cfg.desc}.", "",
             "Commands (run from /tmp with TMPDIR=/tmp; the bench runs from the repository root):", "",
             f"    rocprofv3 --kernel-trace --stats --output-format csv -d <trace> -o run -- {cmd}",
             f"    python3 bench.py --config {cfg.name} --steps {args.steps} --warmup {args.warmup} "
             "--record-patterns <trace>", "",
             "The pattern kernels (`ep_pattern_*`) make the step's memory accesses with none of its arithmetic: "
             "push (x row read, then k scattered FP8-sized row writes per token), gather (k scattered row "
             "reads, then one row write per token; capped as the combine, and uncapped), compact fill and "
             "compact read. Average duration per launch over the whole run (its launches cycle through the "
             "rotated sets); rate = the bytes each launch moves / average duration.", "",
             "| kernel | calls | avg us | bytes per launch | TB/s |", "|---|---|---|---|---|"]
    for key in PATTERN_KERNELS:
        if key not in rows or key == "k_copy":
            continue
        calls, us = rows[key]
        lines.append(f"| `{key}` | {calls} | {us:.2f} | {nb[key]} | {nb[key] / (us * 1e-6) / 1e12:.3f} |")
    if "k_layout_dispatch" in rows and "k_pattern_push" in rows and "k_combine" in rows and \
            "k_pattern_gather" in rows:
        rd = (nb["k_layout_dispatch"] / rows["k_layout_dispatch"][1]) / (nb["k_pattern_push"] / rows["k_pattern_push"][1])
        rc = (nb["k_combine"] / rows["k_combine"][1]) / (nb["k_pattern_gather"] / rows["k_pattern_gather"][1])
        lines += ["", f"Fused layout+dispatch rate / push pattern rate: {rd:.3f}. "
                      f"Combine rate / gather pattern rate: {rc:.3f}."]
    lines += ["", f"Kernel sources: sha256 prefix {source_sha()} (ep_kernels.hip, ep_api.hip, ep_internal.h)."]
    path = os.path.join(PROFILES, f"{cfg.name}_access_patterns.md")
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    return path


def traffic_key(cfg, args):
    return cfg.name + ("_low_latency" if args.ll else "_dedup" if args.dedup else "") + \
        ("_separate" if args.separate else "")


def mode_flags(args):
    return "".join(f" --{n}" for n in ("ll", "dedup", "separate") if getattr(args, n))


def record_traffic(args, cfg, nb_copy):
    fetch = _per_kernel(_csv_rows(args.record_traffic[0], "counter_collection.csv"), "Counter_Value")
    write = _per_kernel(_csv_rows(args.record_traffic[1], "counter_collection.csv"), "Counter_Value")
    n = args.steps + args.warmup
    mean = lambda xs: sum(xs) / len(xs)
    # calibration: the copy kernel moves nb_copy bytes in and nb_copy out
    f_copy = mean([v for g, v in fetch["k_copy"]]) * 1024.0
    w_copy = mean([v for g, v in write["k_copy"]]) * 1024.0
    f_scale, w_scale = nb_copy / f_copy, nb_copy / w_copy
    res = {"source_sha": source_sha(), "workload": cfg.name,
           "calibration": {"copy_bytes_each_way": nb_copy, "FETCH_SIZE_bytes": f_copy, "WRITE_SIZE_bytes": w_copy,
                           "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4)}}
    for k in [k for k in KERNELS if k != "k_copy"]:
        # the first n launches in order (the layout's first launch sizes the buffers)
        first = 1 if k == "k_layout" else 0
        fs = [v for g, v in fetch[k]][first:first + n]
        ws = [v for g, v in write[k]][first:first + n]
        if not fs or len(fs) != len(ws):
            continue
        fb, wb = mean(fs) * 1024.0 * f_scale, mean(ws) * 1024.0 * w_scale
        res[k] = {"launches": len(fs), "fetch_bytes": round(fb), "write_bytes": round(wb),
                  "hbm_bytes_per_launch": round(fb + wb)}
    trace = _csv_rows(args.record_traffic[2], "kernel_stats.csv")
    path = os.path.join(PROFILES, "traffic.json")
    try:
        with open(path) as f:
            allres = json.load(f)
    except (OSError, ValueError):
        allres = {}
    allres[traffic_key(cfg, args)] = res
    with open(path, "w") as f:
        json.dump(allres, f, indent=1)
    return res, trace


def write_profile_summaries(args, cfg, res, trace, algo):
    ll = mode_flags(args)
    cmd_bench = (f"python3 bench.py --config {cfg.name}{ll} --steps {args.steps} --warmup {args.warmup} "
                 "--no-cpu-baseline --no-decode" + (" --no-extras" if args.no_extras and not (args.ll or args.dedup) else ""))
    lines = [f"# {cfg.name}: kernel trace and HBM traffic (rocprofv3)", "",
             f"Workload: {cfg.desc}.", "",
             "Commands (run from /tmp with TMPDIR=/tmp; the bench runs from the repository root):", "",
             f"    rocprofv3 --kernel-trace --stats --output-format csv -d <trace> -o run -- {cmd_bench}",
             f"    rocprofv3 --pmc FETCH_SIZE --output-format csv -d <fetch> -o run -- {cmd_bench}",
             f"    rocprofv3 --pmc WRITE_SIZE --output-format csv -d <write> -o run -- {cmd_bench}",
             f"    python3 bench.py --config {cfg.name}{ll} --steps {args.steps} --warmup {args.warmup} "
             "--record-traffic <fetch> <write> <trace>", "",
             "## Kernel statistics (--kernel-trace --stats)", "",
             "| kernel | calls | avg us | min us | max us | share % |", "|---|---|---|---|---|---|"]
    for r in sorted(trace, key=lambda r: -float(r["TotalDurationNs"]))[:12]:
        name = r["Name"].replace("ep::(anonymous namespace)::", "").replace("void ", "")
        name = name.split("(")[0][:60]
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f} |")
    c = res["calibration"]
    lines += ["", "## HBM traffic per launch (--pmc FETCH_SIZE, --pmc WRITE_SIZE)", "",
              f"Calibration: the plain copy kernel moves {c['copy_bytes_each_way']} B each way; "
              f"FETCH_SIZE reads {c['FETCH_SIZE_bytes']:.0f} B and WRITE_SIZE {c['WRITE_SIZE_bytes']:.0f} B "
              f"for it, so the counters are scaled by {c['fetch_scale']} and {c['write_scale']}.", "",
              "| kernel | launches | fetch MB | write MB | HBM MB | algorithmic MB | HBM / algorithmic |",
              "|---|---|---|---|---|---|---|"]
    for k in [k for k in KERNELS if k in res]:
        e = res[k]
        a = algo.get(k)
        ratio = f"{e['hbm_bytes_per_launch'] / a:.3f}" if a else "-"
        amb = f"{a / 1e6:.1f}" if a else "-"
        lines.append(f"| `{k}` | {e['launches']} | {e['fetch_bytes'] / 1e6:.1f} | {e['write_bytes'] / 1e6:.1f} | "
                     f"{e['hbm_bytes_per_launch'] / 1e6:.1f} | {amb} | {ratio} |")
    lines += ["", f"Kernel sources: sha256 prefix {res['source_sha']} (ep_kernels.hip, ep_api.hip, ep_internal.h)."]
    with open(os.path.join(PROFILES, f"{traffic_key(cfg, args)}_kernels_and_traffic.md"), "w") as f:
        f.write("\n".join(lines) + "\n")


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(path, seconds):
    """The oracle as it stands (single-threaded C) on the same workload:
    layout + positions + FP8 dispatch + combine, repeated whole steps until
    about `seconds` of CPU time have elapsed, pinned to one core; each op is
    timed on its own as well (median over the steps)."""
    import numpy as np
    import oracle
    cfg = path.cfg
    wl = path.wl
    orc = oracle.default()
    cap = path.cap
    n = cfg.R * cap
    eo = path.expert_out.view(path.torch.int16).cpu().numpy().view(np.uint16)
    try:
        old_aff = os.sched_getaffinity(0)
        os.sched_setaffinity(0, {sorted(old_aff)[min(1, len(old_aff) - 1)]})
    except (AttributeError, OSError):
        old_aff = None
    steps = 0
    ops = {"layout": [], "positions": [], "dispatch": [], "combine": []}
    t0 = time.perf_counter()
    nk = 0
    while True:
        a = time.perf_counter()
        L = orc.layout(wl.topk_idx, cfg.E, cfg.R, cap)
        b = time.perf_counter()
        pos, _ = orc.positions(wl.topk_idx, L, cfg.E, cfg.R, cap)
        c_ = time.perf_counter()
        orc.dispatch(wl.x, wl.topk_w, pos, n, cfg.use_fp8)
        d_ = time.perf_counter()
        orc.combine(eo, pos, wl.topk_w)
        e_ = time.perf_counter()
        for name, dt in zip(ops, (b - a, c_ - b, d_ - c_, e_ - d_)):
            ops[name].append(dt)
        nk = int((pos >= 0).sum())
        steps += 1
        el = time.perf_counter() - t0
        if el >= seconds or steps >= 50:
            break
    # the backward pair on the last step's positions (bf16 gradients: x as
    # the gradient of the combined tokens, the expert outputs as the rows')
    bwd = {"combine_backward": [], "dispatch_backward": []}
    for _ in range(3):
        a = time.perf_counter()
        orc.combine_backward(wl.x, pos, n)
        b = time.perf_counter()
        orc.dispatch_backward(eo, pos, wl.topk_w)
        bwd["combine_backward"].append(b - a)
        bwd["dispatch_backward"].append(time.perf_counter() - b)
    if old_aff is not None:
        os.sched_setaffinity(0, old_aff)
    d, c, cb = algo_bytes(cfg.T, cfg.k, cfg.H, nk, cfg.use_fp8)
    per_step = el / steps
    bmed = {k: sorted(v)[1] for k, v in bwd.items()}
    return {"value": round((d + c) / per_step / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{steps} whole {cfg.name} steps (layout+positions+dispatch+combine, "
                      f"T={cfg.T}), {per_step * 1e3:.1f} ms/step, single-threaded C oracle on one pinned core; "
                      "then 3 runs of the backward pair",
            "ms_per_step": round(per_step * 1e3, 2),
            "median_ms": {**{k: round(sorted(v)[len(v) // 2] * 1e3, 2) for k, v in ops.items()},
                          **{k: round(v * 1e3, 2) for k, v in bmed.items()}},
            "backward_GBps": round((cb + c) / sum(bmed.values()) / 1e9, 3),
            "host": {"cpu": cpu_model(), "nproc": os.cpu_count()}}


def main():
    args = parse()
    if args.ll and args.dedup:
        raise SystemExit("bench.py: --ll and --dedup are two different steps; pick one")
    if args.ll or args.dedup:
        args.no_extras = True
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (--gpus {args.gpus} requested); "
              "the multi-GPU exchange is not part of it.", file=sys.stderr)
        sys.exit(2)
    from combine_get_dispatch_amd import workloads
    cfg = workloads.CONFIGS[args.config]
    if args.tokens_per_rank:
        # the other reading of "N tokens": N on every source rank, R*N on the GPU
        from dataclasses import replace
        cfg = replace(cfg, T=cfg.T * cfg.R)
    K, W = args.steps, args.warmup
    if args.record_counters:
        # no GPU work: summarize the profiler output of earlier runs of this bench
        print(record_counters(args, cfg))
        return
    if args.record_patterns:
        # no GPU work: summarize the kernel trace of an earlier --patterns-only run
        print(record_patterns(args, cfg))
        return
    if args.record_traffic:
        # no GPU work: summarize the profiler output of an earlier run of this bench
        import numpy as np
        wl = workloads.make_workload(cfg, seed=args.seed, with_x=False)
        N = int((wl.topk_idx >= 0).sum())
        d_b, c_b, _ = algo_bytes(cfg.T, cfg.k, cfg.H, N, cfg.use_fp8)
        # rows of the rank-deduplicated form: distinct (token, destination rank) pairs
        epr = cfg.E // cfg.R
        tk = wl.topk_idx
        t_of = np.repeat(np.arange(cfg.T), cfg.k).reshape(tk.shape)
        Nd = int(np.unique((t_of * cfg.R + tk // epr)[tk >= 0]).size)
        dd_b, dp_b, dc_b = dedup_bytes(cfg.T, cfg.k, cfg.H, Nd, N, cfg.use_fp8)
        if args.dedup:  # the step's combine reads the deduplicated rows
            c_b = dc_b
        res, trace = record_traffic(args, cfg, (c_b // 2) // 16 * 16)  # the copy the bench ran
        write_profile_summaries(args, cfg, res, trace, {"k_layout_dispatch": d_b, "k_dispatch": d_b, "k_combine": c_b,
                                                        "k_ll_dispatch": d_b, "k_dispatch_dedup": dd_b,
                                                        "k_layout_dispatch_dedup": dd_b, "k_prereduce": dp_b})
        print(json.dumps(res))
        return

    import torch
    from combine_get_dispatch_amd import ep
    ep.load()
    torch.cuda.set_device(0)
    main_path = Path(cfg, args.seed, torch, ep, workloads)
    fused = not args.separate and not args.ll and not args.dedup

    def step_of(path):
        """(ops, buffer, form object) of one step on `path`'s inputs."""
        if args.ll:
            f = LlPath(path, torch, ep, workloads, args.seed)
            return [f.dispatch_op, f.combine_op], f.buf, f
        if args.dedup:
            f = DedupPath(path, torch, ep, workloads, args.seed)
            return ([f.layout_op, f.dispatch_op, f.prereduce_op, f.combine_op] if args.separate else
                    [f.fused_op, f.prereduce_op, f.combine_op]), f.buf, f
        return ([path.fused_op, path.combine_op] if fused else
                [path.layout_op, path.dispatch_op, path.combine_op]), path.buf, path

    # the ops of the step, by name, in order
    op_names = (["ll_dispatch", "combine"] if args.ll else
                (["layout", "dispatch"] if args.separate else ["layout_dispatch"]) + ["prereduce", "combine"]
                if args.dedup else
                ["layout_dispatch", "combine"] if fused else ["layout", "dispatch", "combine"])

    # Rotated buffers: consecutive steps use independent sets of inputs and
    # buffers, enough sets that together they exceed the 256 MB memory-side
    # cache many times over (about 2 GiB), so no step finds the previous
    # step's rows there; a single set is timed beside them.
    d0, c0, _ = algo_bytes(cfg.T, cfg.k, cfg.H, cfg.T * cfg.k, cfg.use_fp8)
    n_sets = max(1, min(16, -(-(2 << 30) // max(d0 + c0, 1))))
    sets = [main_path] + [Path(cfg, args.seed + i, torch, ep, workloads) for i in range(1, n_sets)]
    steps = [step_of(q) for q in sets]
    main_ops, step_buf, form = steps[0]
    llp = form if args.ll else None
    dedp = form if args.dedup else None
    # eager launches with events around every op (the per-kernel durations,
    # pooled over the sets; the step itself with --eager)
    op_stats = []
    eager_ms, per_op = timed_rotating(torch, [st[0] for st in steps], K, W, op_stats)
    op_ms = dict(zip(op_names, per_op))
    com_ms = op_ms["combine"]
    if args.eager:
        ms, ms_events, per_graph = eager_ms, eager_ms, 0
    else:
        ms, ms_events, per_graph = graph_rotating(torch, [st[0] for st in steps], K, W)
    one_ms, _, _ = graph_step_timed(torch, main_ops, K, W)  # a single set, for comparison
    for _, b, _ in steps:
        st = b.status()
        if st:
            raise SystemExit(f"bench: device status {st} on {cfg.name}")
    if llp is not None:
        N = int((llp.handle.pos >= 0).sum().item())
    elif dedp is not None:
        N = dedp.rows()
    else:
        N = main_path.kept_slots()
    d_bytes, c_bytes, cb_bytes = algo_bytes(cfg.T, cfg.k, cfg.H, N, cfg.use_fp8)
    p_bytes = 0
    if dedp is not None:  # N: deduplicated rows; the pre-reduction reads the kept slots' outputs
        d_bytes, p_bytes, c_bytes = dedup_bytes(cfg.T, cfg.k, cfg.H, N, int((main_path.topk >= 0).sum().item()),
                                                cfg.use_fp8)
    value = (d_bytes + p_bytes + c_bytes) / (ms * 1e-3) / 1e9
    # the dominant kernel's duration: K of its launches, cycling through the
    # rotated sets, back to back between two HIP events on its stream (no
    # event between launches, whose queue latency would be counted, and no
    # data left in the MALL by the launch before); events around each launch
    # in the timed eager steps, and K launches on one set, are reported beside
    kern_ms = back_to_back_rotating(torch, [st[0][-1] for st in steps], K, W)
    achieved = c_bytes / (kern_ms * 1e-3) / 1e9
    comb_ms = stream_timed(torch, torch.cuda.current_stream(), main_ops[-1:], K, W)
    traffic = measured_traffic("k_combine", traffic_key(cfg, args))

    out = {
        "metric": "dispatch+combine HBM GB/s & % of peak, 4096x7168 top-8; us at 128 tokens",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 dispatch / bf16 rows / fp32 accumulate" if cfg.use_fp8 else "bf16 / fp32 accumulate",
        "data": "synthetic (seeded)",
        "config": {"workload": cfg.name, "tokens": cfg.T,
                   "tokens_read_as": "per source rank" if args.tokens_per_rank else "per GPU",
                   "hidden": cfg.H, "experts": cfg.E,
                   "ranks_simulated": cfg.R, "topk": cfg.k, "routing": cfg.routing,
                   "fp8_dispatch": cfg.use_fp8, "cap_rows": step_buf.cap_rows, "kept_slots": N,
                   "step": ("low-latency dispatch launch, then combine" if llp is not None else
                            "rank-deduplicated layout, dispatch, expert-side pre-reduction, combine (four launches)"
                            if dedp is not None and args.separate else
                            "fused rank-deduplicated layout+dispatch launch, expert-side pre-reduction, combine"
                            if dedp is not None else
                            "fused layout+dispatch launch, then combine" if fused
                            else "layout, dispatch, combine (three launches)") +
                           ("; eager launches" if args.eager else
                            f"; HIP graph of {per_graph} steps, replayed {K // max(per_graph, 1)} times") +
                           f"; {n_sets} rotated sets of inputs and buffers"},
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "kernel": "k_combine", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes_per_launch": c_bytes,
                     "launch_us": round(kern_ms * 1e3, 2),
                     "timing": f"{K} launches back to back between two HIP events, cycling through the "
                               f"{len(steps)} rotated sets",
                     "events_around_each_launch": {"launch_us": round(com_ms * 1e3, 2),
                                                   "achieved": round(c_bytes / (com_ms * 1e-3) / 1e9, 1)},
                     "back_to_back_one_set": {"launch_us": round(comb_ms * 1e3, 2),
                                              "achieved": round(c_bytes / (comb_ms * 1e-3) / 1e9, 1)}},
        "kernels": {},
        "step_us_by_events": round(ms_events * 1e3, 2),
        "single_buffer_set": {"us_per_step_graph": round(one_ms * 1e3, 2),
                              "GBps": round((d_bytes + p_bytes + c_bytes) / (one_ms * 1e-3) / 1e9, 1),
                              "note": "one set of buffers reused every step: part of it stays in the MALL"},
        "eager_step": {"us_per_step": round(eager_ms * 1e3, 2),
                       "GBps": round((d_bytes + p_bytes + c_bytes) / (eager_ms * 1e-3) / 1e9, 1)},
    }
    if dedp is not None:
        out["config"]["bytes"] = {"dispatch": d_bytes, "prereduce": p_bytes, "combine": c_bytes,
                                  "note": "value counts all three: the pre-reduction is part of this step"}
    op_bytes = {"layout_dispatch": d_bytes, "dispatch": d_bytes, "ll_dispatch": d_bytes, "prereduce": p_bytes}
    for name, t_ms in op_ms.items():
        if name == "combine":
            out["kernels"]["combine"] = {"us": round(t_ms * 1e3, 2), "bytes": c_bytes, "GBps": round(achieved, 1)}
        elif name == "layout":
            out["kernels"]["layout"] = {"us": round(t_ms * 1e3, 2)}
        else:
            b_ = op_bytes[name]
            out["kernels"][name] = {"us": round(t_ms * 1e3, 2), "bytes": b_,
                                    "GBps": round(b_ / (t_ms * 1e-3) / 1e9, 1)}
    for kname, (p10, p50, p90) in zip(op_names, op_stats):
        out["kernels"][kname].update({"p10_us": round(p10 * 1e3, 2), "median_us": round(p50 * 1e3, 2),
                                      "p90_us": round(p90 * 1e3, 2)})
    if not args.no_extras:
        # the same eager steps, each after a 1 GiB write that evicts the
        # 256 MB memory-side cache (outside the events)
        scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        fl = []
        for i in range(W + K):
            scratch.fill_(i & 255)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for op in main_ops:
                op()
            e1.record()
            if i >= W:
                fl.append((e0, e1))
        torch.cuda.synchronize()
        fl_ms = sorted(a.elapsed_time(b) for a, b in fl)
        out["eager_step_after_mall_flush"] = {"median_us": round(fl_ms[K // 2] * 1e3, 2),
                                              "mean_us": round(sum(fl_ms) / K * 1e3, 2),
                                              "GBps_median": round((d_bytes + c_bytes) / (fl_ms[K // 2] * 1e-3) / 1e9,
                                                                   1)}
        del scratch
    print(f"# main: {ms * 1e3:.1f} us/step  " +
          "  ".join(f"{k} {v['us']:.1f}" for k, v in out["kernels"].items()) + " us", file=sys.stderr, flush=True)

    if (args.patterns_only or not args.no_extras) and fused and not (args.ll or args.dedup) and \
            cfg.H % 1024 == 0 and cfg.k <= 8:
        pf = pattern_floors(torch, ep, steps, sets, K, W, d_bytes, c_bytes, N)
        if args.patterns_only:
            print(json.dumps(pf))
            return
        out["access_pattern_floors"] = pf
        print(f"# access patterns: combine {pf['combine']['us']:.1f} us vs gather {pf['gather_capped']['us']:.1f}"
              + (f"; layout+dispatch {pf['layout_dispatch']['us']:.1f} us vs push {pf['push']['us']:.1f}; "
                 f"step at the patterns' rates {pf['step_at_pattern_rates_us']:.1f} us" if "push" in pf else ""),
              file=sys.stderr, flush=True)
    for q, (_, b, f) in zip(sets, steps):
        if f is not q:
            b.close()
    for q in sets[1:]:
        q.buf.close()
    del sets, steps, form, llp, dedp
    if not args.no_extras:
        # the other form of the same step, on the same buffers
        p = main_path
        if fused:
            ams, (l_, d_, c_) = timed(torch, [p.layout_op, p.dispatch_op, p.combine_op], K, W)
            out["separate_calls"] = {"us_per_step": round(ams * 1e3, 2), "layout_us": round(l_ * 1e3, 2),
                                     "dispatch_us": round(d_ * 1e3, 2), "combine_us": round(c_ * 1e3, 2)}
        else:
            ams, (ld_, c_) = timed(torch, [p.fused_op, p.combine_op], K, W)
            out["fused_launch"] = {"us_per_step": round(ams * 1e3, 2), "layout_dispatch_us": round(ld_ * 1e3, 2),
                                   "combine_us": round(c_ * 1e3, 2)}
        if p.buf.status():
            raise SystemExit(f"bench: device status {p.buf.status()} on {cfg.name}")

    if not args.no_extras:
        # backward pair on the same handle (bf16 gradients)
        p = main_path
        n = p.buf.num_rows
        gy = workloads.device_normal_bf16((cfg.T, cfg.H), seed=args.seed + 202)
        grows = torch.empty((n, cfg.H), dtype=torch.bfloat16, device="cuda")
        gx = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device="cuda")
        bms, (cb_ms, db_ms) = timed(torch, [lambda: p.buf.combine_backward(gy, p.handle, out=grows),
                                            lambda: p.buf.dispatch_backward(p.expert_out, p.handle, p.w, out=gx)],
                                    K, W)
        out["backward"] = {"workload": cfg.name, "us_per_step": round(bms * 1e3, 2),
                           "combine_backward": {"us": round(cb_ms * 1e3, 2),
                                                "GBps": round(cb_bytes / (cb_ms * 1e-3) / 1e9, 1)},
                           "dispatch_backward": {"us": round(db_ms * 1e3, 2),
                                                 "GBps": round(c_bytes / (db_ms * 1e-3) / 1e9, 1)},
                           "GBps": round((cb_bytes + c_bytes) / (bms * 1e-3) / 1e9, 1)}
        del grows, gx, gy
    # plain streaming copy of the combine's byte count (attainable
    # bandwidth; also the counters' calibration in profiled runs)
    nb = (c_bytes // 2) // 16 * 16
    src = torch.empty(nb, dtype=torch.uint8, device="cuda")
    dst = torch.empty(nb, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    cms, (copy_ms,) = timed(torch, [lambda: ep.copy_bytes(src, dst)], K, W)
    out["copy_reference"] = {"bytes_moved": 2 * nb, "us": round(copy_ms * 1e3, 2),
                             "GBps": round(2 * nb / (copy_ms * 1e-3) / 1e9, 1)}
    del src, dst
    if not args.no_extras:
        # rank-deduplicated exchange on the same inputs, over rotated sets as
        # the main step: one row per (token, destination rank), the
        # expert-side pre-reduction of each row's expert outputs, and the
        # combine of the reduced rows. Like for like, this step takes x to
        # the combined tokens as the per-expert step does; its exchange alone
        # (the two launches that cross ranks across GPUs) is timed beside it.
        dq = [main_path] + [Path(cfg, args.seed + i, torch, ep, workloads) for i in range(1, n_sets)]
        dps = [DedupPath(q, torch, ep, workloads, args.seed + i) for i, q in enumerate(dq)]
        full = [[f.fused_op, f.prereduce_op, f.combine_op] for f in dps]
        g_ms = graph_rotating(torch, full, K, W)[0]
        ex_ms = graph_rotating(torch, [[f.fused_op, f.combine_op] for f in dps], K, W)[0]
        e_ms, (ld_, pr_, c_) = timed_rotating(torch, full, K, W)
        g4_ms = graph_rotating(torch, [[f.layout_op, f.dispatch_op, f.prereduce_op, f.combine_op] for f in dps],
                               K, W)[0]
        for f in dps:
            if f.buf.status():
                raise SystemExit(f"bench: device status {f.buf.status()} on {cfg.name} (dedup)")
        Nd = dps[0].rows()
        dd, dpre, dc = dedup_bytes(cfg.T, cfg.k, cfg.H, Nd, N, cfg.use_fp8)
        out["dedup"] = {"workload": cfg.name, "rows": Nd, "rows_per_expert_path": N, "cap_rows": dps[0].cap,
                        "rotated_sets": len(dps),
                        "step": "fused deduplicated layout+dispatch, expert-side pre-reduction, combine of the "
                                "reduced rows (HIP graph)",
                        "us_per_step_graph": round(g_ms * 1e3, 2), "bytes": dd + dpre + dc,
                        "GBps_graph": round((dd + dpre + dc) / (g_ms * 1e-3) / 1e9, 1),
                        "per_expert_step_us": round(ms * 1e3, 2),
                        "time_vs_per_expert_step": round(g_ms / ms, 3),
                        "four_launches_us_per_step_graph": round(g4_ms * 1e3, 2),
                        "us_per_step_eager": round(e_ms * 1e3, 2),
                        "exchange_only": {"us_per_step_graph": round(ex_ms * 1e3, 2), "bytes": dd + dc,
                                          "time_vs_per_expert_step": round(ex_ms / ms, 3),
                                          "note": "fused dispatch + combine: what crosses ranks across GPUs; "
                                                  "one GPU's HBM also carries the pre-reduction"},
                        "layout_dispatch": {"us": round(ld_ * 1e3, 2), "bytes": dd,
                                            "GBps": round(dd / (ld_ * 1e-3) / 1e9, 1),
                                            "frac": round(dd / (ld_ * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
                        "prereduce": {"us": round(pr_ * 1e3, 2), "bytes": dpre,
                                      "GBps": round(dpre / (pr_ * 1e-3) / 1e9, 1),
                                      "frac": round(dpre / (pr_ * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
                        "combine": {"us": round(c_ * 1e3, 2), "bytes": dc,
                                    "GBps": round(dc / (c_ * 1e-3) / 1e9, 1),
                                    "frac": round(dc / (c_ * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}}
        print(f"# dedup: {g_ms * 1e3:.1f} us/step with pre-reduction ({ex_ms * 1e3:.1f} exchange only), "
              f"rows {Nd} of {N}", file=sys.stderr, flush=True)
        for f in dps:
            f.buf.close()
        for q in dq[1:]:
            q.buf.close()
        del dps, dq, full
        torch.cuda.empty_cache()

    if not args.no_extras and cfg.T // cfg.R <= 256:
        # the low-latency form at this shape: same rows and bytes, fixed
        # per-(expert, source) regions, no look-back
        lp = LlPath(main_path, torch, ep, workloads, args.seed)
        ops = [lp.dispatch_op, lp.combine_op]
        le_ms, (lld_, llc_) = timed(torch, ops, K, W)
        lg_ms, _, _ = graph_step_timed(torch, ops, K, W)
        if lp.buf.status():
            raise SystemExit(f"bench: device status {lp.buf.status()} on {cfg.name} (low latency)")
        out["low_latency"] = {"workload": cfg.name, "us_per_step_graph": round(lg_ms * 1e3, 2),
                              "GBps_graph": round((d_bytes + c_bytes) / (lg_ms * 1e-3) / 1e9, 1),
                              "us_per_step_eager": round(le_ms * 1e3, 2),
                              "dispatch": {"us": round(lld_ * 1e3, 2),
                                           "GBps": round(d_bytes / (lld_ * 1e-3) / 1e9, 1)},
                              "combine_us": round(llc_ * 1e3, 2),
                              "receive_rows": lp.buf.num_rows}
        print(f"# low latency at {cfg.name}: {lg_ms * 1e3:.1f} us/step graph", file=sys.stderr, flush=True)
        lp.buf.close()
        del lp

    if not args.no_extras:
        out["cu_cap_overlap"] = cu_cap_overlap(torch, ep, main_path, K, W)
        print("# overlap: " + json.dumps(out["cu_cap_overlap"]), file=sys.stderr, flush=True)

    if not args.no_extras and cfg.name == "prefill" and not (args.ll or args.dedup or args.tokens_per_rank):
        # the other full-size workloads: the skewed routing (the metric's
        # second case) and the large BF16 one with its backward pair, each
        # the fused step over rotated sets replayed from a HIP graph, as above
        out["other_workloads"] = {}
        for wname in ("skewed", "large"):
            wcfg = workloads.CONFIGS[wname]
            wd0, wc0, _ = algo_bytes(wcfg.T, wcfg.k, wcfg.H, wcfg.T * wcfg.k, wcfg.use_fp8)
            wn = max(1, min(16, -(-(2 << 30) // max(wd0 + wc0, 1))))
            wps = [Path(wcfg, args.seed + i, torch, ep, workloads) for i in range(wn)]
            wms, _, _ = graph_rotating(torch, [[q.fused_op, q.combine_op] for q in wps], K, W)
            wN = wps[0].kept_slots()
            wd, wc, wcb = algo_bytes(wcfg.T, wcfg.k, wcfg.H, wN, wcfg.use_fp8)
            entry = {"us_per_step": round(wms * 1e3, 2), "GBps": round((wd + wc) / (wms * 1e-3) / 1e9, 1),
                     "pct_of_hbm_peak": round(100.0 * (wd + wc) / (wms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                     "tokens": wcfg.T, "ranks_simulated": wcfg.R, "routing": wcfg.routing,
                     "fp8_dispatch": wcfg.use_fp8, "kept_slots": wN, "cap_rows": wps[0].cap, "rotated_sets": wn}
            if wcfg.backward:
                q = wps[0]
                gy = workloads.device_normal_bf16((wcfg.T, wcfg.H), seed=args.seed + 303)
                grows = torch.empty((q.buf.num_rows, wcfg.H), dtype=torch.bfloat16, device="cuda")
                gx = torch.empty((wcfg.T, wcfg.H), dtype=torch.bfloat16, device="cuda")
                bms, (cb_ms, db_ms) = timed(torch, [lambda: q.buf.combine_backward(gy, q.handle, out=grows),
                                                    lambda: q.buf.dispatch_backward(q.expert_out, q.handle, q.w,
                                                                                    out=gx)], K, W)
                entry["backward"] = {"us_per_step": round(bms * 1e3, 2),
                                     "combine_backward_us": round(cb_ms * 1e3, 2),
                                     "dispatch_backward_us": round(db_ms * 1e3, 2),
                                     "GBps": round((wcb + wc) / (bms * 1e-3) / 1e9, 1)}
                del gy, grows, gx
            for q in wps:
                if q.buf.status():
                    raise SystemExit(f"bench: device status {q.buf.status()} on {wname}")
                q.buf.close()
            del wps
            torch.cuda.empty_cache()
            out["other_workloads"][wname] = entry
            print(f"# {wname}: {entry['us_per_step']:.1f} us/step, {entry['GBps']:.0f} GB/s", file=sys.stderr,
                  flush=True)

    if not args.no_extras and not args.no_decode:
        # decode latency: 128 tokens (one rank's share) and the 8-rank group.
        # The step is launch-bound, so it is captured in a HIP graph and
        # replayed; eager per-op event times (host launch gaps included) are
        # reported beside it.
        K = args.steps
        dec = {}
        for name in ("decode_rank", "decode"):
            dcfg = workloads.CONFIGS[name]
            dp = Path(dcfg, args.seed, torch, ep, workloads)
            ops3 = [dp.layout_op, dp.dispatch_op, dp.combine_op]
            ops2 = [dp.fused_op, dp.combine_op]
            g_us, g_wall = graph_timed(torch, ops2 if fused else ops3, max(K, 200), W)
            g3_us, _ = graph_timed(torch, ops3, max(K, 200), W)
            dms, (ld_, c_) = timed(torch, ops2, max(K, 100), W)
            dst_ = dp.buf.status()
            dd, dc, _ = algo_bytes(dp.cfg.T, dp.cfg.k, dp.cfg.H, dp.kept_slots(), True)
            lp = LlPath(dp, torch, ep, workloads, args.seed)
            ll_ops = [lp.dispatch_op, lp.combine_op]
            ll_us, _ = graph_timed(torch, ll_ops, max(K, 200), W)
            _, (lld_, llc_) = timed(torch, ll_ops, max(K, 100), W)
            ll_st = lp.buf.status()
            lp.buf.close()
            del lp
            # rotated sets (about 1 GiB of step data together, at most 16),
            # as for the main step: no step finds the previous one's data in
            # the memory-side cache
            dd0, dc0, _ = algo_bytes(dcfg.T, dcfg.k, dcfg.H, dcfg.T * dcfg.k, True)
            nrot = max(1, min(16, -(-(1 << 30) // (dd0 + dc0))))
            rot = [dp] + [Path(dcfg, args.seed + i, torch, ep, workloads) for i in range(1, nrot)]
            r_us = graph_rotating(torch, [[q.fused_op, q.combine_op] if fused else
                                          [q.layout_op, q.dispatch_op, q.combine_op] for q in rot],
                                  max(K, 200), W)[1] * 1e3
            lrot = [LlPath(q, torch, ep, workloads, args.seed, init_rows=False) for q in rot]
            lr_us = graph_rotating(torch, [[f.dispatch_op, f.combine_op] for f in lrot], max(K, 200), W)[1] * 1e3
            for f in lrot:
                ll_st |= f.buf.status()
                f.buf.close()
            for q in rot[1:]:
                dst_ |= q.buf.status()
                q.buf.close()
            del rot, lrot
            dec[name] = {"tokens": dp.cfg.T, "rotated_sets": nrot,
                         "us_per_step_graph_rotated": round(r_us, 2),
                         "us_per_step_graph": round(g_us, 2),
                         "us_per_step_graph_wall": round(g_wall, 2),
                         "GBps_graph": round((dd + dc) / (g_us * 1e-6) / 1e9, 1),
                         "us_per_step_graph_three_launches": round(g3_us, 2),
                         "us_per_step_eager": round(dms * 1e3, 2),
                         "eager_layout_dispatch_us": round(ld_ * 1e3, 2),
                         "eager_combine_us": round(c_ * 1e3, 2), "status": dst_,
                         "low_latency": {"us_per_step_graph_rotated": round(lr_us, 2),
                                         "us_per_step_graph": round(ll_us, 2),
                                         "GBps_graph": round((dd + dc) / (ll_us * 1e-6) / 1e9, 1),
                                         "eager_dispatch_us": round(lld_ * 1e3, 2),
                                         "eager_dispatch_GBps": round(dd / (lld_ * 1e-3) / 1e9, 1),
                                         "eager_combine_us": round(llc_ * 1e3, 2), "status": ll_st}}
            dp.buf.close()
            del dp
        out["decode"] = dec
        # the pages' decode setting runs their low-latency kernels: the
        # headline latency is that path's, with rotated sets like the main
        # step (the normal path's and the single-set figures are beside it)
        out["us_at_128_tokens"] = dec["decode_rank"]["low_latency"]["us_per_step_graph_rotated"]
        out["us_at_128_tokens_normal_path"] = dec["decode_rank"]["us_per_step_graph_rotated"]

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(main_path, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

"""Benchmark of the fused rank-partial sum + residual add + RMSNorm on one MI355X.

Headline: W=4 H=2048 T=4096 (the largest token count of the page's validation
sweep, "[TLERaw] Add NVSHMEM allreduce RMSNorm tutorial", FlagTree PR #1122,
section Correctness: world size 4, hidden 2048, BF16, tokens 1 ... 4096).  A step
is one arrms_fused call (rank sum, residual add, RMSNorm) on one batch of T rows.
The metric is achieved HBM bandwidth: algorithmic bytes 2*T*H*(W+3) + 2*H (read W
partials and the residual, write residual_out and norm_out, read the weight once)
per call, divided by the time per call; also reported as a fraction of the 8 TB/s
HBM3E peak, and as microseconds per call for T = 1, 16, 64, 128, 256, 1024, 4096.

Inputs are resident in HBM before timing starts.  Calls walk through a 4.4 GiB
pool of distinct input/output sets (10 slots of 16384 rows; far more than the
256 MB Infinity Cache), so repeated calls cannot be served from cache.  Points at
T = 4096, 8192, 16384 (beyond the metric's range) separate the per-call fixed time
from the kernel's streaming rate.

`--workload large_hidden` (W=8 T=8192 H=8192), `--workload ragged_outliers`
(W=8 T=16383 H=5120, 1% outliers) or `--workload odd_rows` (W=4 T=4096 H=2047, the
scalar kernel's path) times those shapes instead, headline only.  Any
shape can be timed the same way (rotating pool, oracle parity check, CPU baseline,
JSON) with `--world/--tokens/--hidden/--eps/--x-sigma/--outlier-p/--seed`, which
replace the named workload's values (the page's harness, section Implementation 6,
likewise takes configurable token shapes).

Timing: `value`/`ms_per_step` are host wall clock over the K timed calls between two
synchronisations; `roofline` uses HIP events on the launch stream over the same calls.
The `ceiling` section times the library's most read-heavy kernel (the rank sum alone,
W=8 and W=16) on the same pool as what this GPU streams, and reports the fused
headline as a fraction of it.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "achieved HBM GB/s (% of peak) and µs/call, W=4 H=2048 at T=1..4096"
SWEEP_T = [1, 16, 64, 128, 256, 1024, 4096]
# Beyond the metric's range, to separate the per-call fixed time from the streaming rate.
FIT_T = [4096, 8192, 16384]
POOL_ROWS = 16384
POOL_SLOTS = 10
# what decides the headline launch: the fused kernels and their device helpers, the
# host planner that picks variant, lane layout and XCD runs, and the argument packing
KERNEL_SRC = [os.path.join(ROOT, "residual_add_rmsnorm_arrms_amd", "csrc", f)
              for f in ("arrms_device.h", "arrms_kernels.hip", "arrms_api.cpp", "arrms_internal.h")]
# workloads the benchmark can time (--workload); the default is the metric's own
BENCH_WORKLOADS = ("prefill", "large_hidden", "ragged_outliers", "odd_rows")


def traffic_file(wl) -> str:
    return os.path.join(ROOT, "profiles", "traffic_%s_w%d_h%d_t%d.json" % (wl.name, wl.world, wl.hidden, wl.tokens))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of the kernel, planner and argument-packing source without comments and blank
    lines: what the counters were measured on (a comment edit leaves it unchanged, a code
    edit does not)."""
    import re
    text = "".join(open(f).read() for f in KERNEL_SRC)
    text = re.sub(r"//[^\n]*", "", text)
    code = "\n".join(line.rstrip() for line in text.splitlines() if line.strip())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def algorithmic_bytes(W, T, H):
    return 2 * T * H * (W + 3) + 2 * H


def pool_slots(torch, slot_bytes):
    """Slots of a rotating pool: POOL_SLOTS when they fit in half the GPU's memory, else as
    many as fit (at least 2, so that consecutive calls never share buffers)."""
    total = torch.cuda.get_device_properties(0).total_memory
    n = min(POOL_SLOTS, int(0.5 * total // slot_bytes))
    if n < 2:
        raise SystemExit("bench.py: two pool slots of %.1f GiB do not fit this GPU" % (slot_bytes / 2 ** 30))
    return n


class Pool:
    """Slots (POOL_SLOTS, fewer for very large shapes), each holding W partials, residual,
    residual_out and norm_out of [rows, H] BF16 in one device allocation (the input rows
    repeated to fill `rows`).  A call with T rows uses rows [j*T, (j+1)*T) of one slot, so
    successive calls touch fresh memory."""

    def __init__(self, torch, x, res, w, rows=None):
        W, T_in, H = x.shape
        T = rows or T_in
        self.W, self.T, self.H = W, T, H
        dev = torch.device("cuda", 0)
        self.tensor_elems = T * H
        self.slots = pool_slots(torch, (W + 3) * T * H * 2)
        self.slot = torch.empty((self.slots, W + 3, T, H), dtype=torch.bfloat16, device=dev)
        xd, rd = x.to(dev), res.to(dev)
        for r0 in range(0, T, T_in):
            n = min(T_in, T - r0)
            self.slot[0, :W, r0:r0 + n].copy_(xd[:, :n])
            self.slot[0, W, r0:r0 + n].copy_(rd[:n])
        del xd, rd
        for s in range(1, self.slots):
            self.slot[s, :W + 1].copy_(self.slot[0, :W + 1])
        self.weight = w.to(dev)
        torch.cuda.synchronize()
        self.base = self.slot.data_ptr()

    @property
    def nbytes(self):
        return self.slot.numel() * 2

    def reduced_ptr(self, base, T, j, s):
        """Address of the reduced-output rows of set (j, s) in a [slots, rows, H] buffer."""
        return base + s * self.tensor_elems * 2 + j * T * self.H * 2

    def sets(self, T, max_sets=8192):
        """Pointer sets (partials, residual, residual_out, norm_out) for T-row calls: up to
        max_sets distinct ones, cycling through the slots first."""
        per_slot = min(self.T // T, max(1, max_sets // self.slots))
        out = []
        for j in range(per_slot):
            for s in range(self.slots):
                slot = self.base + s * (self.W + 3) * self.tensor_elems * 2
                off = j * T * self.H * 2
                t = lambda k: slot + k * self.tensor_elems * 2 + off
                out.append(([t(r) for r in range(self.W)], t(self.W), t(self.W + 1), t(self.W + 2)))
        return out


class ReduceCaller:
    """Pre-marshalled arrms_reduce calls: W partials taken from the pool's partial and
    residual tensors of consecutive slots, the output into a separate scratch area."""

    def __init__(self, A, handle, pool, W, T, out_base, stream):
        lib = A.load()
        self.fn = lib.arrms_reduce
        vp = ctypes.c_void_p
        per_slot = min(pool.T // T, max(1, 8192 // pool.slots))
        inputs_per_slot = pool.W + 1
        self.args = []
        te = pool.tensor_elems * 2
        for j in range(per_slot):
            for s in range(pool.slots):
                parts = []
                for r in range(W):
                    slot = (s + r // inputs_per_slot) % pool.slots
                    parts.append(pool.base + slot * (pool.W + 3) * te + (r % inputs_per_slot) * te + j * T * pool.H * 2)
                out = pool.reduced_ptr(out_base, T, j, s)
                self.args.append((vp(handle), (vp * W)(*parts), W, T, pool.H, vp(out)))
        self.stream = vp(stream)
        self.i = 0

    def __call__(self):
        a = self.args[self.i]
        self.i = (self.i + 1) % len(self.args)
        rc = self.fn(*a, self.stream)
        if rc:
            raise RuntimeError("arrms_reduce returned %d" % rc)


class Caller:
    """Pre-marshalled ctypes arguments, so the host side of a call costs little."""

    def __init__(self, A, handle, sets, W, T, H, weight_ptr, eps, stream):
        lib = A.load()
        self.fn = lib.arrms_fused
        vp = ctypes.c_void_p
        self.args = []
        for parts, res, ro, no in sets:
            arr = (vp * W)(*parts)
            self.args.append((vp(handle), arr, W, T, H, vp(res), vp(weight_ptr), ctypes.c_float(eps), vp(ro), vp(no)))
        self.stream = vp(stream)
        self.i = 0

    def __call__(self):
        a = self.args[self.i]
        self.i = (self.i + 1) % len(self.args)
        rc = self.fn(*a, self.stream)
        if rc:
            raise RuntimeError("arrms_fused returned %d" % rc)


def time_back_to_back(torch, call, K):
    """K calls between two synchronisations: (wall ms per call, GPU-event ms per call)."""
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(s)
    for _ in range(K):
        call()
    e1.record(s)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return (t1 - t0) * 1e3 / K, e0.elapsed_time(e1) / K


def time_per_launch(torch, call, K):
    """Duration of each of K launches from an event pair around it, on the launch stream."""
    s = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record(s)
        call()
        b.record(s)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def time_isolated(torch, call, K):
    """Each call alone: synchronise, event, call, event, synchronise (includes launch latency)."""
    s = torch.cuda.current_stream()
    out = []
    for _ in range(K):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(s)
        call()
        b.record(s)
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b))
    return out


def time_graph(torch, call, calls_per_graph, replays, flush=None):
    """calls_per_graph calls captured in one HIP graph, replayed; ms per call.  With
    `flush`, it runs before every replay, outside the timed interval of that replay
    (events around each replay), so that no replay finds its data in the caches."""
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        saved = call.stream
        call.stream = ctypes.c_void_p(side.cuda_stream)
        call()  # warm up on a side stream before capture
        call.stream = saved
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    saved = call.stream
    with torch.cuda.graph(g):
        call.stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        for _ in range(calls_per_graph):
            call()
    call.stream = saved
    g.replay()
    torch.cuda.synchronize()
    if flush is not None:
        total = 0.0
        for _ in range(replays):
            flush()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            total += e0.elapsed_time(e1)
        del g
        return total / (replays * calls_per_graph)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (replays * calls_per_graph)
    del g
    return ms


def launch_floor_graph_us(torch, calls=100, replays=10):
    """GPU time per launch of a one-element kernel replayed from a HIP graph: the floor
    under any kernel's decode latency on this GPU (context for the T=1 sweep point)."""
    t = torch.zeros(1, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        t.add_(1)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            t.add_(1)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (calls * replays)


def pct(xs, q):
    xs = sorted(xs)
    return xs[min(len(xs) - 1, max(0, int(round(q / 100.0 * (len(xs) - 1)))))]


def copy_context(torch, nbytes):
    """Plain device-to-device copy of nbytes (read nbytes + write nbytes): context, not the denominator."""
    n = nbytes // 2
    a = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1.0)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b
    return {"bytes_per_copy": 2 * n * 2, "ms": ms, "GB_s": 2 * n * 2 / (ms * 1e-3) / 1e9}


def copy_same_bytes(torch, nbytes, pairs=10, reps=200):
    """A plain device-to-device copy moving the fused call's algorithmic bytes (nbytes/2 read,
    nbytes/2 written), rotating over `pairs` source/destination pairs so that, like the
    fused calls, successive copies touch fresh memory.  Context for the headline."""
    n = nbytes // 4  # BF16 elements per copy: n*2 bytes read + n*2 written = nbytes
    src = torch.empty((pairs, n), dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1.0)
    for i in range(2 * pairs):
        dst[i % pairs].copy_(src[i % pairs])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        dst[i % pairs].copy_(src[i % pairs])
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return {"bytes_per_copy": 4 * n, "pairs": pairs, "us": ms * 1e3, "GB_s": 4 * n / (ms * 1e-3) / 1e9}


def torch_streams(torch, nbytes=1 << 30, sets=4, reps=30):
    """Same-box references from PyTorch's own kernels, each over `sets` rotating sets of
    about `nbytes` of traffic per call (4 GiB in all, far beyond the 256 MB Infinity
    Cache): a pure read (sum of a BF16 tensor into binary32), two reads and a write
    (add), one read and a write (copy).  GB/s counts the bytes each must move."""
    n = nbytes // 2  # BF16 elements per tensor
    out = {}
    a = torch.ones((sets, n), dtype=torch.bfloat16, device="cuda")
    acc = torch.empty(sets, dtype=torch.float32, device="cuda")

    def timed(fn, moved):
        for i in range(2 * sets):
            fn(i % sets)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(reps):
            fn(i % sets)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        return {"bytes": moved, "us": ms * 1e3, "GB_s": moved / (ms * 1e-3) / 1e9,
                "frac_of_peak": moved / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    out["read_sum"] = timed(lambda i: torch.sum(a[i], dim=0, dtype=torch.float32, out=acc[i]), 2 * n)
    del acc
    b = torch.ones((sets, n // 2), dtype=torch.bfloat16, device="cuda")
    c = torch.empty((sets, n // 2), dtype=torch.bfloat16, device="cuda")
    half = n // 2
    out["add_2r1w"] = timed(lambda i: torch.add(a[i, :half], b[i], out=c[i]), 3 * 2 * half)
    out["copy_1r1w"] = timed(lambda i: c[i].copy_(b[i]), 2 * 2 * half)
    del a, b, c
    torch.cuda.empty_cache()
    for k, v in out.items():
        log("torch %s: %.1f us, %.0f GB/s (%.1f%% of 8 TB/s)" % (k, v["us"], v["GB_s"], 100 * v["frac_of_peak"]))
    return out


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.machine()


def cpu_baseline(x, res, w, eps, budget_s):
    """The oracle (scalar C) on whole prefill calls: single-threaded for up to budget_s, then with
    the rows split over the host threads for up to budget_s / 2."""
    import oracle
    import synth
    xb, rb, wb = synth.bits(x), synth.bits(res), synth.bits(w)
    W, T, H = xb.shape
    times = []
    t_start = time.perf_counter()
    ref = None
    while True:
        t0 = time.perf_counter()
        ref = oracle.fused(xb, rb, wb, eps)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start >= budget_s or len(times) >= 200:
            break
    med = statistics.median(times)
    # the same oracle with the row range split over host threads (rows are independent)
    try:
        nthreads = min(16, len(os.sched_getaffinity(0)))
    except AttributeError:
        nthreads = min(16, os.cpu_count() or 1)
    ttimes = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        oracle.fused(xb, rb, wb, eps, threads=nthreads)
        ttimes.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start >= budget_s / 2 or len(ttimes) >= 200:
            break
    tmed = statistics.median(ttimes)
    threaded = {"value": algorithmic_bytes(W, T, H) / tmed / 1e9, "unit": "GB/s", "cores": nthreads,
                "ms_per_call": tmed * 1e3, "repetitions": len(ttimes),
                "sample": "the same whole call, rows split into %d contiguous ranges, one host thread each"
                          % nthreads}
    return ref, {
        "value": algorithmic_bytes(W, T, H) / med / 1e9,
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": "whole W=%d H=%d T=%d call (all rows), %d repetitions, median %.1f ms, single thread"
                  % (W, H, T, len(times), med * 1e3),
        "ms_per_call": med * 1e3,
        "cpu": cpu_model(),
        "host_threads_available": os.cpu_count(),
        "threaded": threaded,
    }


def traffic_record(wl, plan):
    """DRAM bytes per launch measured by rocprofv3 for workload wl, or None unless they were
    taken on the current kernel, planner and argument-packing source and on the same launch
    plan as this run's."""
    path = traffic_file(wl)
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_sha256_16") != kernel_source_hash() or rec.get("plan") != plan:
        return None
    return rec


class Ctx:
    """What the optional benchmark sections share: the prefill pool and its handle."""

    def __init__(self, torch, A, synth, op, pool, W, H, eps, stream):
        self.torch, self.A, self.synth, self.op, self.pool = torch, A, synth, op, pool
        self.W, self.H, self.eps, self.stream = W, H, eps, stream
        self.cu = torch.cuda.get_device_properties(0).multi_processor_count

    def caller(self, t):
        return Caller(self.A, self.op.handle, self.pool.sets(t), self.W, t, self.H, self.pool.weight.data_ptr(),
                      self.eps, self.stream)

    def flush(self):
        """Stream 1 GiB through memory that no call uses (a 512 MiB device copy), so that the
        256 MB Infinity Cache holds none of the pool's data afterwards."""
        if not hasattr(self, "_flush_buf"):
            self._flush_buf = self.torch.empty((2, 256 * 2 ** 20), dtype=self.torch.bfloat16, device="cuda")
        self._flush_buf[1].copy_(self._flush_buf[0])

    def plan(self, t):
        s, W = self.pool.slot, self.W
        return self.op.plan(s[0, :W, :t], s[0, W, :t], self.pool.weight, self.eps, s[0, W + 1, :t], s[0, W + 2, :t])


VARIANT_NAMES = {1: "row", 2: "splith", 3: "scalar"}


def sweep_tokens(ctx):
    """Sweep over T: back-to-back, per-launch, isolated and graph replay with data coming
    from HBM (each leg starts after a cache flush and its calls take distinct buffers, the
    graph's 100 calls too, with a flush before every replay), then back-to-back and graph
    replay on one set of buffers repeated (hot: inputs in the caches)."""
    torch, W, H = ctx.torch, ctx.W, ctx.H
    sweep = []
    for t in SWEEP_T:
        c = ctx.caller(t)
        p = ctx.plan(t)
        for _ in range(100):
            c()
        k = 2000 if t <= 1024 else 1000
        ctx.flush()
        wall, gpu = time_back_to_back(torch, c, k)
        ctx.flush()
        d = time_per_launch(torch, c, 300)
        ctx.flush()
        iso = time_isolated(torch, c, 100)
        gr = time_graph(torch, c, 100, 10, flush=ctx.flush)
        # the same call repeated on one set of buffers (inputs and outputs stay in the caches)
        hot = Caller(ctx.A, ctx.op.handle, ctx.pool.sets(t)[:1], W, t, H, ctx.pool.weight.data_ptr(), ctx.eps,
                     ctx.stream)
        for _ in range(100):
            hot()
        _, gpu_hot = time_back_to_back(torch, hot, k)
        gr_hot = time_graph(torch, hot, 100, 10)
        b = algorithmic_bytes(W, t, H)
        row = {"T": t, "variant": VARIANT_NAMES[p["variant"]], "grid": p["grid"],
               "block": p["block"], "bytes": b,
               "us_back_to_back_wall": wall * 1e3, "us_back_to_back_gpu": gpu * 1e3,
               "us_event_pair_p50": pct(d, 50) * 1e3, "us_event_pair_p90": pct(d, 90) * 1e3,
               "us_event_pair_p99": pct(d, 99) * 1e3,
               "us_isolated_p50": pct(iso, 50) * 1e3, "us_graph_replay": gr * 1e3,
               "us_back_to_back_gpu_hot": gpu_hot * 1e3, "us_graph_replay_hot": gr_hot * 1e3,
               "GB_s_back_to_back": b / (gpu * 1e-3) / 1e9,
               "GB_s_graph": b / (gr * 1e-3) / 1e9}
        row["frac_peak_back_to_back"] = row["GB_s_back_to_back"] / HBM_PEAK_GBS
        sweep.append(row)
        log("T=%5d %-6s b2b %.2f us (%.0f GB/s, %.1f%%), event pair p50 %.2f us, isolated %.2f us, "
            "graph %.2f us; one hot set: b2b %.2f us, graph %.2f us" % (
                t, row["variant"], row["us_back_to_back_gpu"], row["GB_s_back_to_back"],
                100 * row["frac_peak_back_to_back"], row["us_event_pair_p50"], row["us_isolated_p50"],
                row["us_graph_replay"], row["us_back_to_back_gpu_hot"], row["us_graph_replay_hot"]))
    return sweep


def fixed_and_streaming(ctx):
    """Per-call fixed time and streaming rate: least-squares line through the
    back-to-back GPU time at T = 4096, 8192, 16384 (same kernel, same layout)."""
    pts = []
    for t in FIT_T:
        c = ctx.caller(t)
        for _ in range(50):
            c()
        _, g = time_back_to_back(ctx.torch, c, 500)
        pts.append((t, g * 1e3))
    n = len(pts)
    mt = sum(p[0] for p in pts) / n
    mu = sum(p[1] for p in pts) / n
    slope = sum((p[0] - mt) * (p[1] - mu) for p in pts) / sum((p[0] - mt) ** 2 for p in pts)
    icpt = mu - slope * mt
    row_bytes = 2 * ctx.H * (ctx.W + 3)
    fit = {"points_us": [{"T": t, "us": u} for t, u in pts], "fixed_us_per_call": icpt,
           "us_per_row": slope, "streaming_GB_s": row_bytes / (slope * 1e-6) / 1e9,
           "streaming_frac_of_peak": row_bytes / (slope * 1e-6) / 1e9 / HBM_PEAK_GBS}
    log("fit over T=%s: fixed %.2f us per call, streaming %.0f GB/s (%.1f%% of peak)" % (
        FIT_T, icpt, fit["streaming_GB_s"], 100 * fit["streaming_frac_of_peak"]))
    return fit


def fusion_and_rank_sum(ctx, T, nbytes, fused_ms):
    """The page's two-stage form (rank sum kernel, then the epilogue as a one-rank fused
    call through a BF16 `reduced` tensor) against the fused call; then the rank sum
    alone over sizes and W (reads W partials, writes reduced)."""
    torch, A, op, pool, W, H = ctx.torch, ctx.A, ctx.op, ctx.pool, ctx.W, ctx.H
    red_pool = torch.empty((pool.slots, pool.T, H), dtype=torch.bfloat16, device="cuda")
    rcall = ReduceCaller(A, op.handle, pool, W, T, red_pool.data_ptr(), ctx.stream)
    per_slot = len(pool.sets(T)) // pool.slots
    epi_sets = [([pool.reduced_ptr(red_pool.data_ptr(), T, i // pool.slots, i % pool.slots)], st[1], st[2], st[3])
                for i, st in enumerate(pool.sets(T))]
    assert len(epi_sets) == per_slot * pool.slots
    ecall = Caller(A, op.handle, epi_sets, 1, T, H, pool.weight.data_ptr(), ctx.eps, ctx.stream)

    def two_stage():
        rcall()
        ecall()
    for _ in range(50):
        two_stage()
    _, ts_ms = time_back_to_back(torch, two_stage, 1000)
    _, red_ms = time_back_to_back(torch, rcall, 1000)
    _, epi_ms = time_back_to_back(torch, ecall, 1000)
    ts_bytes = nbytes + 2 * 2 * T * H  # plus writing and re-reading `reduced`
    fusion = {"workload": "W=%d T=%d H=%d" % (W, T, H), "fused_us": fused_ms * 1e3, "two_stage_us": ts_ms * 1e3,
              "reduce_kernel_us": red_ms * 1e3, "epilogue_kernel_us": epi_ms * 1e3,
              "two_stage_bytes": ts_bytes, "fused_bytes": nbytes,
              "fused_speedup": ts_ms / fused_ms}
    log("fusion: fused %.2f us vs two-stage %.2f us (reduce %.2f + epilogue %.2f): %.2fx" % (
        fused_ms * 1e3, ts_ms * 1e3, red_ms * 1e3, epi_ms * 1e3, ts_ms / fused_ms))
    reduce_sweep = []
    for w_ in (2, 4, 8):
        for t in (16, 256, 4096):
            c = ReduceCaller(A, op.handle, pool, w_, t, red_pool.data_ptr(), ctx.stream)
            for _ in range(50):
                c()
            _, ms = time_back_to_back(torch, c, 1000)
            b = 2 * t * H * (w_ + 1)
            reduce_sweep.append({"W": w_, "T": t, "H": H, "bytes": b, "us": ms * 1e3,
                                 "GB_s": b / (ms * 1e-3) / 1e9})
            log("reduce only W=%d T=%5d: %.2f us, %.0f GB/s" % (w_, t, ms * 1e3, b / (ms * 1e-3) / 1e9))
    del red_pool
    return fusion, reduce_sweep


def forced_variants(ctx):
    """Each variant forced on the same shapes (the automatic choice is one of them)."""
    A, op = ctx.A, ctx.op
    variants = []
    for v in (A.ARRMS_VARIANT_ROW, A.ARRMS_VARIANT_SPLITH, A.ARRMS_VARIANT_SCALAR):
        name = VARIANT_NAMES[v]
        op.set_variant(v)
        for t in (1, 16, 128, 4096):
            c = ctx.caller(t)
            p = ctx.plan(t)
            for _ in range(50):
                c()
            _, g = time_back_to_back(ctx.torch, c, 1000 if t <= 128 else 300)
            b = algorithmic_bytes(ctx.W, t, ctx.H)
            variants.append({"variant": name, "T": t, "grid": p["grid"], "block": p["block"],
                             "kernels": p["kernels"], "us_back_to_back_gpu": g * 1e3,
                             "GB_s": b / (g * 1e-3) / 1e9})
            log("variant %-6s T=%5d: %.2f us (%.0f GB/s), grid %d x %d, %d kernel(s)" % (
                name, t, g * 1e3, b / (g * 1e-3) / 1e9, p["grid"], p["block"], p["kernels"]))
    op.set_variant(A.ARRMS_VARIANT_AUTO)
    return variants


def store_policy(ctx, tokens=(4096, 16384), rounds=2):
    """residual_out written with streaming stores (the default) against write-back stores
    (tuning residual_out_store=2) on the prefill pool's rotating buffers: back-to-back GPU
    time, the two policies interleaved, the best of `rounds` each."""
    torch, A, op = ctx.torch, ctx.A, ctx.op
    out = []
    for t in tokens:
        best = {}
        for _ in range(rounds):
            for store, name in ((1, "streaming"), (2, "write_back")):
                op.set_tuning(residual_out_store=store)
                c = ctx.caller(t)
                for _ in range(30):
                    c()
                _, g = time_back_to_back(torch, c, 300 if t <= 4096 else 100)
                best[name] = min(best.get(name, 1e9), g * 1e3)
        op.set_tuning()
        b = algorithmic_bytes(ctx.W, t, ctx.H)
        rec = {"W": ctx.W, "T": t, "H": ctx.H}
        for name, us in best.items():
            rec[name + "_us"] = us
            rec[name + "_frac_of_peak_gpu_events"] = b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS
        out.append(rec)
        log("residual_out stores W=%d T=%d H=%d: streaming %.2f us, write-back %.2f us" % (
            ctx.W, t, ctx.H, best["streaming"], best["write_back"]))
    return out


def kernarg_preload(ctx, tokens=(1024, 4096), rounds=3):
    """Kernels with preloaded arguments (the automatic choice from 16 MiB per call)
    against the same kernels taking one argument block (tuning kernarg_preload=1), on
    the prefill pool's rotating buffers: back-to-back GPU time, interleaved, the best of
    `rounds` each."""
    torch, op = ctx.torch, ctx.op
    out = []
    for t in tokens:
        best = {}
        for _ in range(rounds):
            for mode, name in ((0, "preloaded"), (1, "argument_block")):
                op.set_tuning(kernarg_preload=mode)
                c = ctx.caller(t)
                for _ in range(30):
                    c()
                _, g = time_back_to_back(torch, c, 300 if t <= 4096 else 100)
                best[name] = min(best.get(name, 1e9), g * 1e3)
        op.set_tuning()
        plan = ctx.plan(t)
        b = algorithmic_bytes(ctx.W, t, ctx.H)
        rec = {"W": ctx.W, "T": t, "H": ctx.H, "automatic_kernarg_preload": plan["kernarg_preload"]}
        for name, us in best.items():
            rec[name + "_us"] = us
            rec[name + "_frac_of_peak_gpu_events"] = b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS
        out.append(rec)
        log("kernel arguments W=%d T=%d H=%d: preloaded %.2f us, one argument block %.2f us" % (
            ctx.W, t, ctx.H, best["preloaded"], best["argument_block"]))
    return out


def line_offset_rows(ctx, shapes=((1, 16384, 2040), (4, 4096, 6000)), rounds=3):
    """Rows whose stride is not a multiple of 128 bytes (H % 64 != 0): the automatic plan
    (the scalar kernel, its lanes rotated onto whole lines) against the row kernel forced.
    Each shape on its own rotating pool (its first 256 rows of seeded inputs repeated),
    back-to-back GPU time, the two interleaved, the best of `rounds` each."""
    torch, A = ctx.torch, ctx.A
    out = []
    for W, T, H in shapes:
        wl = ctx.synth.WORKLOADS["prefill"].with_(world=W, tokens=min(T, 256), hidden=H, seed=700 + W)
        x, r, w = ctx.synth.make_inputs(wl)
        lpool = Pool(torch, x, r, w, rows=T)
        del x, r
        lop = A.FusedReduceResidualRMSNorm(max_world=W, max_tokens=T, max_hidden=H, device=0)
        lctx = Ctx(torch, A, ctx.synth, lop, lpool, W, H, wl.eps, ctx.stream)
        rec = {"W": W, "T": T, "H": H}
        best = {}
        for _ in range(rounds):
            for variant, name in ((A.ARRMS_VARIANT_AUTO, "auto"), (A.ARRMS_VARIANT_ROW, "row")):
                lop.set_variant(variant)
                rec[name + "_variant"] = VARIANT_NAMES[lctx.plan(T)["variant"]]
                c = lctx.caller(T)
                for _ in range(30):
                    c()
                _, g = time_back_to_back(torch, c, 300 if T <= 4096 else 100)
                best[name] = min(best.get(name, 1e9), g * 1e3)
        b = algorithmic_bytes(W, T, H)
        for name, us in best.items():
            rec[name + "_us"] = us
            rec[name + "_frac_of_peak_gpu_events"] = b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS
        out.append(rec)
        log("line-offset rows W=%d T=%d H=%d: automatic (%s) %.2f us, row kernel %.2f us" % (
            W, T, H, rec["auto_variant"], best["auto"], best["row"]))
        lop.close()
        del lpool
        torch.cuda.empty_cache()
    return out


def reduce_offsets(ctx, W=4, T=4096):
    """The rank sum alone at W=4 T=4096 H=2048 with its tensors placed at byte offsets:
    every tensor at the same offset (16-byte loads after a short head) and the output
    at an offset the partials do not share (8-, 4- and 2-byte loads).  Back-to-back GPU
    time over the prefill pool's buffers: a call reads rows of partials 0..W-1 of a slot,
    so an offset read ends at most 14 bytes into the next tensor of the same slot."""
    torch, A, op, pool, H = ctx.torch, ctx.A, ctx.op, ctx.pool, ctx.H
    fn = A.load().arrms_reduce
    vp = ctypes.c_void_p
    te = pool.tensor_elems * 2
    # one spare row per output slot: an offset output still ends inside its slot
    out = torch.empty((pool.slots, pool.T + 1, H), dtype=torch.bfloat16, device="cuda")
    res = []
    for part_off, out_off in ((0, 0), (2, 2), (0, 8), (0, 4), (0, 2)):
        calls = []
        for j in range(pool.T // T):
            for sl in range(pool.slots):
                base = pool.base + sl * (pool.W + 3) * te + j * T * H * 2
                parts = [base + r * te + part_off for r in range(W)]
                o = out[sl].data_ptr() + j * T * H * 2 + out_off
                calls.append(((vp * W)(*parts), vp(o)))
        rc, p = A.arrms_plan_reduce(ctx.cu, None, 16, pool.T, H, [c for c in calls[0][0]], W, T, H, calls[0][1].value)
        state = {"i": 0}

        def call():
            a = calls[state["i"] % len(calls)]
            state["i"] += 1
            r = fn(vp(op.handle), a[0], W, T, H, a[1], vp(ctx.stream))
            if r:
                raise RuntimeError("arrms_reduce returned %d" % r)
        for _ in range(20):
            call()
        _, ms = time_back_to_back(torch, call, 300)
        b = 2 * T * H * (W + 1)
        res.append({"W": W, "T": T, "H": H, "partials_offset": part_off, "reduced_offset": out_off,
                    "elems_per_load": p["elems_per_load"], "us": ms * 1e3, "GB_s": b / (ms * 1e-3) / 1e9})
        log("rank sum W=%d T=%d, partials +%d B, output +%d B: %d-byte loads, %.2f us, %.0f GB/s" % (
            W, T, part_off, out_off, 2 * p["elems_per_load"], ms * 1e3, b / (ms * 1e-3) / 1e9))
    del out
    return res


def scalar_widths(ctx, T=4096):
    """The scalar variant (rows the 16-byte kernels cannot take) at W=4 T=4096: rows of
    H = 2044, 2046 and 2047 elements (8-, 4- and 2-byte loads chosen automatically) on
    the prefill pool's buffers read with that row length, and H = 2048 forced through
    the scalar kernel with each load width.  Back-to-back GPU time."""
    torch, A, op, W = ctx.torch, ctx.A, ctx.op, ctx.W
    sets = ctx.pool.sets(T)  # row length below 2048 stays inside each 2048-element row slot
    out = []
    cases = [(2044, None), (2046, None), (2047, None), (2048, 4), (2048, 2), (2048, 1)]
    for H, elems in cases:
        if elems:
            op.set_variant(A.ARRMS_VARIANT_SCALAR)
            op.set_tuning(scalar_elems=elems)
        c = Caller(A, op.handle, sets, W, T, H, ctx.pool.weight.data_ptr(), ctx.eps, ctx.stream)
        s0 = ctx.pool.slot[0]
        view = lambda k: s0[k].view(-1)[:T * H].view(T, H)
        p = op.plan([view(r) for r in range(W)], view(W), ctx.pool.weight[:H], ctx.eps, view(W + 1), view(W + 2))
        for _ in range(50):
            c()
        _, g = time_back_to_back(torch, c, 500)
        op.set_variant(A.ARRMS_VARIANT_AUTO)
        op.set_tuning()
        b = algorithmic_bytes(W, T, H)
        out.append({"W": W, "T": T, "H": H, "forced": bool(elems), "variant": VARIANT_NAMES[p["variant"]],
                    "elems_per_load": p["elems_per_load"], "us": g * 1e3, "GB_s": b / (g * 1e-3) / 1e9,
                    "frac_of_peak_gpu_events": b / (g * 1e-3) / 1e9 / HBM_PEAK_GBS})
        log("scalar W=%d T=%d H=%d%s: %d-byte loads, %.2f us, %.0f GB/s" % (
            W, T, H, " (forced)" if elems else "", 2 * p["elems_per_load"], g * 1e3, b / (g * 1e-3) / 1e9))
    return out


def world_sweep(ctx, T=4096, worlds=(1, 2, 3, 4, 6, 8, 12, 16)):
    """The fused call at H=2048 T=4096 across rank counts (the shapes of other
    tensor-parallel degrees): back-to-back GPU time and achieved bandwidth, each W
    on its own 10-slot rotating pool (automatic plan)."""
    torch, A, H = ctx.torch, ctx.A, ctx.H
    out = []
    for W in worlds:
        wl = ctx.synth.WORKLOADS["prefill"].with_(world=W, tokens=T, seed=500 + W)
        x, r, w = ctx.synth.make_inputs(wl)
        wpool = Pool(torch, x, r, w, rows=T)
        del x, r
        wop = A.FusedReduceResidualRMSNorm(max_world=W, max_tokens=T, max_hidden=H, device=0)
        wctx = Ctx(torch, A, ctx.synth, wop, wpool, W, H, wl.eps, ctx.stream)
        c = wctx.caller(T)
        p = wctx.plan(T)
        for _ in range(30):
            c()
        _, g = time_back_to_back(torch, c, 500)
        b = algorithmic_bytes(W, T, H)
        out.append({"W": W, "T": T, "H": H, "us": g * 1e3, "GB_s": b / (g * 1e-3) / 1e9,
                    "frac_of_peak_gpu_events": b / (g * 1e-3) / 1e9 / HBM_PEAK_GBS,
                    "vec_per_thread": p["vec_per_thread"],
                    "threads_per_row": p["threads_per_row"], "xcd_chunk": p["xcd_chunk"]})
        log("W=%2d T=%d H=%d: %.2f us, %.0f GB/s (%.1f%%)" % (W, T, H, g * 1e3, b / (g * 1e-3) / 1e9,
                                                           100 * out[-1]["frac_of_peak_gpu_events"]))
        wop.close()
        del wpool
        torch.cuda.empty_cache()
    return out


def read_ceiling(ctx, achieved_gbs, T=16384, worlds=(8, 16)):
    """What this GPU streams with the library's own most read-heavy kernel: the rank sum
    alone (arrms_reduce, W reads per write) at T=16384 H=2048, back-to-back GPU time.
    Each call reads W distinct 64 MiB input tensors of the prefill pool (its 10 slots hold
    50), consecutive calls take disjoint ones, and outputs rotate over 10 buffers, so no
    call finds its inputs in the 256 MB Infinity Cache.  The fused headline's achieved
    bandwidth is reported as a fraction of the faster of these rates."""
    torch, A, op, pool, H = ctx.torch, ctx.A, ctx.op, ctx.pool, ctx.H
    assert pool.T >= T
    fn = A.load().arrms_reduce
    vp = ctypes.c_void_p
    te = pool.tensor_elems * 2
    inputs = [pool.base + s * (pool.W + 3) * te + k * te for s in range(pool.slots) for k in range(pool.W + 1)]
    out = torch.empty((pool.slots, T, H), dtype=torch.bfloat16, device="cuda")
    res = {}
    for W in worlds:
        calls = []
        for i in range(len(inputs)):
            parts = [inputs[(i * W + r) % len(inputs)] for r in range(W)]
            calls.append((vp(op.handle), (vp * W)(*parts), W, T, H, vp(out[i % pool.slots].data_ptr()),
                          vp(ctx.stream)))
        state = {"i": 0}

        def call():
            a = calls[state["i"]]
            state["i"] = (state["i"] + 1) % len(calls)
            rc = fn(*a)
            if rc:
                raise RuntimeError("arrms_reduce returned %d" % rc)
        for _ in range(20):
            call()
        _, ms = time_back_to_back(torch, call, 200)
        b = 2 * T * H * (W + 1)
        res["reduce_W%d" % W] = {"W": W, "T": T, "H": H, "bytes": b, "us": ms * 1e3, "GB_s": b / (ms * 1e-3) / 1e9,
                                 "frac_of_peak": b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        log("ceiling: rank sum alone W=%d T=%d H=%d: %.2f us, %.0f GB/s (%.1f%% of 8 TB/s)" % (
            W, T, H, ms * 1e3, b / (ms * 1e-3) / 1e9, 100 * b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS))
    del out
    best = max(v["GB_s"] for v in res.values())
    res["ceiling_GB_s"] = best
    res["fused_headline_GB_s"] = achieved_gbs
    res["fused_frac_of_ceiling"] = achieved_gbs / best
    log("fused headline %.0f GB/s = %.1f%% of that ceiling" % (achieved_gbs, 100 * achieved_gbs / best))
    return res


def splith_crossover(ctx):
    """Where split-H pays: long rows (W=8 H=8192, 180 KB of traffic per row) at decode
    token counts, row vs split-H vs the automatic choice, HIP-graph replay (GPU time per
    call; 10 rotating sets of 128 rows, 230 MB)."""
    torch, A = ctx.torch, ctx.A
    lw = ctx.synth.WORKLOADS["large_hidden"].with_(tokens=128)
    lx, lr, lwt = ctx.synth.make_inputs(lw)
    lpool = Pool(torch, lx, lr, lwt, rows=128)
    del lx, lr
    lop = A.FusedReduceResidualRMSNorm(max_world=lw.world, max_tokens=128, max_hidden=lw.hidden, device=0)
    lctx = Ctx(torch, A, ctx.synth, lop, lpool, lw.world, lw.hidden, lw.eps, ctx.stream)
    out = []
    for t in (1, 4, 16, 64, 128):
        row = {"W": lw.world, "H": lw.hidden, "T": t}
        for v, name in ((A.ARRMS_VARIANT_AUTO, "auto"), (A.ARRMS_VARIANT_ROW, "row"),
                        (A.ARRMS_VARIANT_SPLITH, "splith")):
            lop.set_variant(v)
            c = lctx.caller(t)
            p = lctx.plan(t)
            for _ in range(20):
                c()
            row["us_graph_" + name] = time_graph(torch, c, 50, 10) * 1e3
            if name == "auto":
                row["auto_variant"] = VARIANT_NAMES[p["variant"]]
        lop.set_variant(A.ARRMS_VARIANT_AUTO)
        out.append(row)
        log("W=8 H=8192 T=%3d graph replay: row %.2f us, split-H %.2f us, auto (%s) %.2f us" % (
            t, row["us_graph_row"], row["us_graph_splith"], row["auto_variant"], row["us_graph_auto"]))
    lop.close()
    del lpool
    return out


# ------------------------------------------------------------ rocprofv3 summaries
def _short_kernel_name(n: str) -> str:
    n = n.replace("void arrms::(anonymous namespace)::", "")
    if n.startswith(("row_kernel", "splith_", "scalar_kernel", "reduce_")):
        n = n[:n.index("(")] if "(" in n else n
    return n[:70]


# Counter passes (one rocprofv3 --pmc run each; at most four TCC counters per run).
# DRAM bytes come from the gfx950 counters that count DRAM reads and writes in
# 32-byte units (a 64-byte request counts 2, a 128-byte read 4).
PMC_PASSES = {
    "dram": ["TCC_EA0_RDREQ_DRAM_32B_sum", "TCC_EA0_WRREQ_WRITE_DRAM_32B_sum", "TCC_EA0_RDREQ_sum",
             "TCC_BUBBLE_sum"],
    "size": ["TCC_EA0_RDREQ_32B_sum", "TCC_EA0_RDREQ_64B_sum", "TCC_EA0_RDREQ_128B_sum", "TCC_EA0_WRREQ_64B_sum"],
    "stall": ["TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum", "TCC_EA0_WRREQ_DRAM_CREDIT_STALL_sum", "TCC_BUSY_sum",
              "TCC_EA0_RDREQ_LEVEL_sum"],
    "fetch": ["FETCH_SIZE"],
    "write": ["WRITE_SIZE"],
}


def pmc_command(workload: str, name: str) -> str:
    flag = "" if workload == "prefill" else " --workload %s" % workload
    return ("timeout -s KILL 300 rocprofv3 --pmc %s --output-format csv -d <run dir>/pmc_%s -o %s -- "
            "python -u bench.py%s --no-cpu --no-sweep --steps 50 --warmup 5"
            % (" ".join(PMC_PASSES[name]), name, name, flag))


def read_counters(path: str) -> dict:
    """{(kernel, grid size): {counter: [value per dispatch]}} from a rocprofv3 counter CSV."""
    import collections
    import csv
    out = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in csv.DictReader(open(path)):
        out[(_short_kernel_name(r["Kernel_Name"]), int(r["Grid_Size"]))][r["Counter_Name"]].append(
            float(r["Counter_Value"]))
    return out


def summarize_profiles(run_dir: str, workload: str, out_dir: str = None) -> None:
    """Write profiles/<kernel>_<workload>.md and profiles/traffic_<workload>.json from
    the rocprofv3 outputs found under run_dir: bench.json and prof_bench/ (kernel trace of
    the benchmark command), pmc_<pass>/ for the counter passes of PMC_PASSES."""
    import collections
    import csv
    import synth
    wl = synth.WORKLOADS[workload]
    W, T, H = wl.world, wl.tokens, wl.hidden
    alg = algorithmic_bytes(W, T, H)
    alg_read, alg_write = 2 * T * H * (W + 1) + 2 * H, 2 * T * H * 2
    sha = kernel_source_hash()
    bench = json.load(open(os.path.join(run_dir, "bench.json")))
    plan = bench["config"]["plan"]
    grid_threads = plan["grid"] * plan["block"]
    flag = "" if workload == "prefill" else " --workload %s" % workload
    trace = collections.defaultdict(list)
    for r in csv.DictReader(open(os.path.join(run_dir, "prof_bench", "bench_kernel_trace.csv"))):
        key = (_short_kernel_name(r["Kernel_Name"]), int(r["Grid_Size_X"]), int(r["Workgroup_Size_X"]))
        trace[key].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    # the headline kernel: the most dispatched library kernel at the headline launch shape
    kname = max((len(v), k) for k, v in trace.items()
                if k[1] == grid_threads and k[2] == plan["block"] and ("kernel<" in k[0] or "kernel_flat<" in k[0]))[1][0]
    head = trace[(kname, grid_threads, plan["block"])]
    kkey = (kname, grid_threads)
    mean = {}
    dispatches = {}
    for name in PMC_PASSES:
        path = os.path.join(run_dir, "pmc_%s" % name, "%s_counter_collection.csv" % name)
        if not os.path.exists(path):
            continue
        c = read_counters(path)[kkey]
        for cn, vals in c.items():
            mean[cn] = statistics.mean(vals)
            dispatches[cn] = len(vals)
    rd = 32 * mean["TCC_EA0_RDREQ_DRAM_32B_sum"]
    wr = 32 * mean["TCC_EA0_WRREQ_WRITE_DRAM_32B_sum"]
    by_size = None
    if "TCC_EA0_RDREQ_128B_sum" in mean:
        by_size = (32 * mean["TCC_EA0_RDREQ_32B_sum"] + 64 * mean["TCC_EA0_RDREQ_64B_sum"] +
                   128 * mean["TCC_EA0_RDREQ_128B_sum"])
    # the derived FETCH_SIZE's own formula on gfx950, from its raw terms
    fetch_formula = (128 * mean["TCC_BUBBLE_sum"] + 64 * (mean["TCC_EA0_RDREQ_sum"] - mean["TCC_BUBBLE_sum"] -
                                                          mean.get("TCC_EA0_RDREQ_32B_sum", 0.0)) +
                     32 * mean.get("TCC_EA0_RDREQ_32B_sum", 0.0))
    stalls = None
    if "TCC_BUSY_sum" in mean:
        busy = mean["TCC_BUSY_sum"]
        stalls = {"tcc_busy_cycles_sum": busy,
                  "read_dram_credit_stall_pct_of_busy": 100 * mean["TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum"] / busy,
                  "write_dram_credit_stall_pct_of_busy": 100 * mean["TCC_EA0_WRREQ_DRAM_CREDIT_STALL_sum"] / busy,
                  "mean_read_requests_in_flight_per_channel": mean["TCC_EA0_RDREQ_LEVEL_sum"] / busy,
                  "mean_read_latency_cycles": mean["TCC_EA0_RDREQ_LEVEL_sum"] / mean["TCC_EA0_RDREQ_sum"]}
    commands = [pmc_command(workload, n) for n in PMC_PASSES]
    base = "%s_w%d_h%d_t%d" % (workload, W, H, T)
    traffic = {
        "kernel": kname, "workload": "W=%d T=%d H=%d (%s), launch grid %d x %d" % (W, T, H, workload, plan["grid"],
                                                                                plan["block"]),
        "plan": plan, "dispatches": dispatches, "counters_mean_per_dispatch": mean,
        "read_bytes_per_launch": rd, "write_bytes_per_launch": wr,
        "algorithmic_read_bytes": alg_read, "algorithmic_write_bytes": alg_write,
        "read_bytes_by_request_size": by_size, "fetch_size_formula_bytes": fetch_formula,
        "algorithmic_bytes_per_launch": alg, "traffic_over_algorithmic": (rd + wr) / alg,
        "stalls": stalls, "kernel_source_sha256_16": sha, "commands": commands,
    }
    out_dir = out_dir or os.path.join(ROOT, "profiles")
    json.dump(traffic, open(os.path.join(out_dir, os.path.basename(traffic_file(wl))), "w"), indent=1)
    cmd_trace = ("cd /tmp && TMPDIR=/tmp rocprofv3 --kernel-trace --stats --output-format csv "
                 "-d <run dir>/prof_bench -o bench -- python -u bench.py" + flag)
    L = ["# %s on W=%d T=%d H=%d (%s) — rocprofv3 summary\n" % (kname, W, T, H, workload),
         "GPU: MI355X (gfx950), one GPU.  Source hash of the kernels, planner and argument packing (sha256[:16] "
         "of the code without comments, as bench.py computes it) = `%s`.  Written by `python bench.py --summarize "
         "<run dir>%s` from the runs below.\n" % (sha, flag),
         "## Kernel trace (same command as the benchmark)\n", "```\n%s\n```\n" % cmd_trace]
    if workload == "prefill":
        L.append("Dispatches grouped by kernel and launch shape (grid in threads). The headline launch is `%s`, grid "
                 "%d x %d threads; other launch shapes come from the token sweep, the forced-variant, split-H, "
                 "rank-sum and ceiling sections and the copy references. Shapes with fewer than 3 dispatches are "
                 "left out.\n" % (kname, plan["grid"], plan["block"]))
    else:
        L.append("Dispatches grouped by kernel and launch shape (grid in threads); the headline launch is `%s`, grid "
                 "%d x %d threads, and `copyBuffer` comes from the copy references. Shapes with fewer than 3 "
                 "dispatches are left out.\n" % (kname, plan["grid"], plan["block"]))
    L += ["| kernel | grid (threads) | block | dispatches | mean us | p50 us | min us | max us |",
          "|---|---|---|---|---|---|---|---|"]
    for (k, gs, bs), v in sorted(trace.items(), key=lambda kv: (-len(kv[1]), kv[0])):
        if len(v) >= 3:
            L.append("| %s | %d | %d | %d | %.2f | %.2f | %.2f | %.2f |" % (
                k, gs, bs, len(v), statistics.mean(v) / 1e3, statistics.median(v) / 1e3, min(v) / 1e3,
                max(v) / 1e3))
    hm = statistics.mean(head) / 1e3
    L.append("\nHeadline launch: mean %.2f us over %d dispatches -> %.1f GB/s algorithmic (%d B per launch); "
             "bench.py reported %.2f us per launch from HIP events over its timed region (%.1f GB/s).\n" % (
                 hm, len(head), alg / (hm * 1e-6) / 1e9, alg, bench["roofline"]["kernel_mean_us"],
                 bench["roofline"]["achieved"]))
    L += ["## HBM traffic from raw TCC counters, one pass per run\n",
          "```\n%s\n```\n" % "\n".join(commands),
          "DRAM bytes are 32 x `TCC_EA0_RDREQ_DRAM_32B_sum` (reads) and 32 x `TCC_EA0_WRREQ_WRITE_DRAM_32B_sum` "
          "(writes): these gfx950 counters count DRAM traffic in 32-byte units, so no calibration factor is "
          "applied.\n",
          "| quantity | per launch | algorithmic |", "|---|---|---|",
          "| DRAM read bytes | %.0f | %d (W partials + residual + weight) |" % (rd, alg_read),
          "| DRAM write bytes | %.0f | %d (residual_out + norm_out) |" % (wr, alg_write),
          "| total / algorithmic | %.4f | 1 |" % ((rd + wr) / alg)]
    if by_size is not None:
        L += ["| read bytes from request sizes (32 x n32 + 64 x n64 + 128 x n128) | %.0f | |" % by_size,
              "| read requests of 32 / 64 / 128 bytes | %.0f / %.0f / %.0f | |" % (
                  mean["TCC_EA0_RDREQ_32B_sum"], mean["TCC_EA0_RDREQ_64B_sum"], mean["TCC_EA0_RDREQ_128B_sum"])]
    L += ["| `TCC_EA0_RDREQ_sum` / `TCC_BUBBLE_sum` | %.0f / %.0f | |" % (mean["TCC_EA0_RDREQ_sum"],
                                                                         mean["TCC_BUBBLE_sum"]),
          "| derived FETCH_SIZE formula from those terms (bytes) | %.0f | |" % fetch_formula]
    if "FETCH_SIZE" in mean and "WRITE_SIZE" in mean:
        L.append("| derived FETCH_SIZE / WRITE_SIZE as rocprofv3 reports them (bytes) | %.0f / %.0f | |" % (
            1024 * mean["FETCH_SIZE"], 1024 * mean["WRITE_SIZE"]))
    if stalls:
        L += ["\n## Memory-side stalls (same kernel)\n", "| quantity | value |", "|---|---|",
              "| read requests stalled on DRAM credits, %% of TCC busy cycles | %.2f |" %
              stalls["read_dram_credit_stall_pct_of_busy"],
              "| write requests stalled on DRAM credits, %% of TCC busy cycles | %.2f |" %
              stalls["write_dram_credit_stall_pct_of_busy"],
              "| mean read requests in flight per TCC channel, over its busy cycles | %.1f |" %
              stalls["mean_read_requests_in_flight_per_channel"],
              "| mean TCC-to-memory read latency, cycles | %.0f |" % stalls["mean_read_latency_cycles"]]
    with open(os.path.join(out_dir, "%s_%s.md" % (kname.split("<")[0], base)), "w") as f:
        f.write("\n".join(L) + "\n")


def workload_from_args(synth, args):
    """The named workload, with any shape or distribution given on the command line
    replacing its own (then named "custom")."""
    wl = synth.WORKLOADS[args.workload]
    over = {k: v for k, v in (("world", args.world), ("tokens", args.tokens), ("hidden", args.hidden),
                              ("eps", args.eps), ("x_sigma", args.x_sigma), ("outlier_p", args.outlier_p),
                              ("seed", args.seed)) if v is not None}
    if not over:
        return wl
    if not (1 <= over.get("world", wl.world) <= 16 and over.get("tokens", wl.tokens) >= 1 and
            1 <= over.get("hidden", wl.hidden) <= 65536 and over.get("eps", wl.eps) >= 0 and
            0 <= over.get("outlier_p", wl.outlier_p) <= 1 and over.get("x_sigma", wl.x_sigma) > 0):
        raise SystemExit("bench.py: shape or distribution out of range: %s" % over)
    return wl.with_(name="custom", **over)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle timing")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline leg")
    ap.add_argument("--no-sweep", action="store_true", help="only the T=4096 headline")
    ap.add_argument("--workload", default="prefill", choices=BENCH_WORKLOADS,
                    help="headline workload (the T sweep, fit, fusion, variant, rank-sum and ceiling sections "
                         "run only for the unmodified prefill workload, the metric's W=4 H=2048 shape)")
    ap.add_argument("--world", type=int, help="W: rank partials (overrides the workload's)")
    ap.add_argument("--tokens", type=int, help="T: token rows (overrides the workload's)")
    ap.add_argument("--hidden", type=int, help="H: hidden size (overrides the workload's)")
    ap.add_argument("--eps", type=float, help="RMSNorm eps (overrides the workload's)")
    ap.add_argument("--x-sigma", type=float, help="standard deviation of the partials (overrides the workload's)")
    ap.add_argument("--outlier-p", type=float, help="fraction of partial entries scaled x100 (overrides)")
    ap.add_argument("--seed", type=int, help="input seed (overrides the workload's)")
    ap.add_argument("--summarize", metavar="RUN_DIR",
                    help="write the profiles/ summary of the workload from rocprofv3 outputs in RUN_DIR and exit")
    args = ap.parse_args()
    if args.summarize:
        summarize_profiles(args.summarize, args.workload)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the partial sums of all ranks are modelled as buffers already "
              "in this GPU's memory, and nothing here uses a second GPU. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import synth
    wl = workload_from_args(synth, args)
    if wl.name != "prefill":
        args.no_sweep = True

    import torch
    import residual_add_rmsnorm_arrms_amd as A

    if not os.path.exists(A.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    torch.cuda.set_device(0)
    props = torch.cuda.get_device_properties(0)
    W, T, H, eps = wl.world, wl.tokens, wl.hidden, wl.eps
    log("generating inputs W=%d T=%d H=%d" % (W, T, H))
    x, res, w = synth.make_inputs(wl)
    # prefill: 16384-row slots, so the T <= 16384 points of the fit also rotate; larger
    # workloads: one call per slot (each slot alone is far beyond the Infinity Cache)
    pool_rows = POOL_ROWS if 4 * T <= POOL_ROWS else T
    pool = Pool(torch, x, res, w, rows=pool_rows)
    log("pool: %d slots, %.2f GiB" % (pool.slots, pool.nbytes / 2 ** 30))
    op = A.FusedReduceResidualRMSNorm(max_world=16, max_tokens=pool_rows, max_hidden=H, device=0)
    stream = torch.cuda.current_stream().cuda_stream

    def caller(t):
        return Caller(A, op.handle, pool.sets(t), W, t, H, pool.weight.data_ptr(), eps, stream)

    # ---- headline: T=4096, K timed steps between synchronisations
    call = caller(T)
    plan = op.plan(pool.slot[0, :W, :T], pool.slot[0, W, :T], pool.weight, eps, pool.slot[0, W + 1, :T],
                   pool.slot[0, W + 2, :T])
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    wall_ms, gpu_ms = time_back_to_back(torch, call, args.steps)
    nbytes = algorithmic_bytes(W, T, H)
    log("headline: %.3f us/call wall, %.3f us/call GPU events" % (wall_ms * 1e3, gpu_ms * 1e3))
    # ---- roofline: kernel time from the events around the timed region (launch stream),
    # i.e. gpu_ms per launch; per-launch event pairs give the spread (each pair adds
    # the events' own overhead, about 2 us, so their mean is not used for the roofline)
    achieved = nbytes / (gpu_ms * 1e-3) / 1e9
    durs = time_per_launch(torch, call, max(200, min(args.steps, 2000)))
    log("per-launch event pairs: p50 %.3f us, p90 %.3f, p99 %.3f; roofline %.1f GB/s" % (
        pct(durs, 50) * 1e3, pct(durs, 90) * 1e3, pct(durs, 99) * 1e3, achieved))

    # correctness of the timed configuration: one set against the oracle
    torch.cuda.synchronize()
    parity = None
    cpu = None
    if not args.no_cpu:
        ref, cpu = cpu_baseline(x, res, w, eps, args.cpu_budget)
        log("cpu oracle: %.2f GB/s (%s); %d threads: %.2f GB/s" % (
            cpu["value"], cpu["sample"], cpu["threaded"]["cores"], cpu["threaded"]["value"]))
        s0 = pool.sets(T)[0]
        A.arrms_fused(op.handle, s0[0], W, T, H, s0[1], pool.weight.data_ptr(), eps, s0[2], s0[3], stream)
        torch.cuda.synchronize()
        ro = synth.bits(pool.slot[0, W + 1, :T].cpu())
        no = synth.bits(pool.slot[0, W + 2, :T].cpu())
        parity = {"residual_out_mismatches": int((ro != ref["residual_out"]).sum()),
                  "norm_out_not_bit_identical": int((no != ref["norm_out"]).sum()),
                  "elements": int(ro.size)}
        log("parity of the timed configuration vs oracle: %s" % parity)

    sweep, fit, fusion, reduce_sweep, variants, splith_regime, worlds = [], None, None, [], [], [], []
    ceiling, scalar, reduce_offs, stores, line_offset, preload = None, [], [], [], [], []
    if not args.no_sweep:
        ctx = Ctx(torch, A, synth, op, pool, W, H, eps, stream)
        ceiling = read_ceiling(ctx, achieved)
        sweep = sweep_tokens(ctx)
        fit = fixed_and_streaming(ctx)
        fusion, reduce_sweep = fusion_and_rank_sum(ctx, T, nbytes, gpu_ms)
        variants = forced_variants(ctx)
        scalar = scalar_widths(ctx)
        reduce_offs = reduce_offsets(ctx)
        stores = store_policy(ctx, tokens=tuple(t for t in (4096, 16384) if t <= pool.T))
        line_offset = line_offset_rows(ctx)
        preload = kernarg_preload(ctx, tokens=tuple(t for t in (1024, 4096) if t <= pool.T))
        splith_regime = splith_crossover(ctx)
        worlds = world_sweep(ctx)

    floor_us = launch_floor_graph_us(torch)
    log("launch floor (one-element kernel, graph replay): %.2f us" % floor_us)
    copy = copy_context(torch, 512 * 2 ** 20)
    log("copy context: %.1f GB/s" % copy["GB_s"])
    streams = torch_streams(torch) if not args.no_sweep else None
    copy_same = copy_same_bytes(torch, nbytes, pairs=max(2, min(10, int(4e9 // nbytes))))
    log("copy of the headline's byte count (%d B, rotating): %.2f us, %.1f GB/s" % (
        copy_same["bytes_per_copy"], copy_same["us"], copy_same["GB_s"]))
    tr = traffic_record(wl, plan)
    op.close()

    value = nbytes / (wall_ms * 1e-3) / 1e9
    out = {
        "metric": METRIC if wl.name == "prefill" else
        "achieved HBM GB/s (%% of peak) and µs/call, W=%d H=%d T=%d" % (W, H, T),
        "value": value,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded SplitMix64/Box-Muller; x~N(0,%g^2)%s, residual~N(0,%g^2), weight~U(%g,%g))" % (
            wl.x_sigma, (", %g%% of x elements scaled x%g" % (100 * wl.outlier_p, wl.outlier_scale))
            if wl.outlier_p else "", wl.residual_sigma, wl.weight_lo, wl.weight_hi),
        "config": {"workload": "%s: W=%d rank partials, T=%d tokens, H=%d, BF16 in/out, eps=%g" % (
                   wl.name, W, T, H, eps),
                   "world": W, "tokens": T, "hidden": H, "io_dtype": "bf16", "accumulate": "f32 rank sum, f64 "
                   "sum of squares", "algorithmic_bytes_per_call": nbytes, "plan": plan,
                   "pool_bytes": pool.nbytes, "parallelism": "1 GPU"},
        "frac_of_peak_wall": value / HBM_PEAK_GBS,
        "us_per_call": wall_ms * 1e3,
        "timing": "value, ms_per_step, us_per_call and frac_of_peak_wall: host wall clock over the K timed "
                  "calls between two synchronisations; roofline: HIP events on the launch stream over the same "
                  "region",
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": (tr["read_bytes_per_launch"] + tr["write_bytes_per_launch"]) if tr else None,
                     "kernel_mean_us": gpu_ms * 1e3, "launches_timed": args.steps,
                     "timing": "HIP events on the launch stream around the K timed launches",
                     "event_pair_p50_us": pct(durs, 50) * 1e3, "event_pair_p90_us": pct(durs, 90) * 1e3,
                     "event_pair_p99_us": pct(durs, 99) * 1e3},
        "cpu_baseline": cpu,
        "parity_vs_oracle": parity,
        "sweep": sweep,
        "fusion": fusion,
        "fixed_and_streaming": fit,
        "reduce_only": reduce_sweep,
        "copy_context": copy,
        "copy_same_bytes": copy_same,
        "torch_streams": streams,
        "variants": variants,
        "scalar_widths": scalar,
        "reduce_offsets": reduce_offs,
        "store_policy": stores,
        "line_offset_rows": line_offset,
        "kernarg_preload": preload,
        "splith_regime": splith_regime,
        "world_sweep": worlds,
        "ceiling": ceiling,
        "launch_floor_graph_us": floor_us,
        "device": {"name": props.name, "compute_units": props.multi_processor_count,
                   "gcn_arch": getattr(props, "gcnArchName", None), "memory_GiB": props.total_memory / 2 ** 30},
        "kernel_source_sha256_16": kernel_source_hash(),
    }
    if tr:
        out["roofline"]["traffic_detail"] = tr
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

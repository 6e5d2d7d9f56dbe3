#!/usr/bin/env python3
"""Benchmark of the ALHR tree-attention path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload t16k]

A step is one pass of the whole prefill path over one batch: tree build and
budget prediction (alhr_prepare: the two share their launches), then the
fused route + attend kernel, i.e. the kernels alhr_forward launches, issued
as its two ABI calls back to back, with fence-free HIP timing events on the
launch stream around the route call.  Untimed auxiliary measurements (the
routing's load counts, the dense baseline, the splitter) run first.  Inputs
are synthetic and resident in HBM before the timed region.  Prints one JSON
line:

  value     routed queries/s of the whole step (B * H * T queries per step)
  roofline  the fused route + attend kernel against vector-instruction issue,
            the bound that limits it (VALU instructions per query from the
            committed SQ counters x queries / the event-timed launch, against
            1024 SIMDs x 2.4 GHz / 4); beside it `hbm` (rocprofv3 FETCH_SIZE +
            WRITE_SIZE bytes past L2, scaled by a plain-copy calibration,
            against 8 TB/s: an upper bound on the HBM share) and
            `bytes_touched` (algorithmic bytes); counter figures are null when
            the committed counters were taken on other source
  cpu_baseline  the single-threaded C oracle on a bounded sample of the same
            workload, pinned to one host core (cpu_baseline_all_cores: the
            same sample with whole pairs spread over up to 16 host threads)
  decode    the decode workload (2^17-position, 64 x 16-head cache; append +
            route + attend per token, 128-token loops) with its HBM roofline
            and a sampled-pair oracle rate (leave out with --no-decode)

--workload decode prints the decode measurement as the line itself.
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

HBM_PEAK_GBS = 8000.0
INT8_MFMA_PEAK_TOPS = 5000.0   # MI355X dense int8 MFMA, 5.0 POP/s
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "route_attend_t16k_counters.txt")
PROFILE_DECODE_COUNTERS = os.path.join(ROOT, "profiles", "decode_t131072_counters.txt")
ROUTE_SOURCES = [os.path.join(ROOT, "learned_tree_routed_amd", "csrc", f)
                 for f in ("route.hip", "device.h", "append.h")]


def route_source_sha():
    """Hash of the route kernel's source with comments and blank lines
    dropped, and of the extra compiler flags route.hip is built with, so that
    editing a comment does not orphan the recorded counters while any change
    to the code or to how it is compiled does."""
    import re
    from learned_tree_routed_amd.build import EXTRA
    h = hashlib.sha256()
    for p in ROUTE_SOURCES:
        text = open(p, encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        lines = [ln.rstrip() for ln in text.splitlines() if ln.strip()]
        h.update("\n".join(lines).encode())
    flags = EXTRA.get("route.hip", [])
    if flags:
        h.update(("\nflags: " + " ".join(flags)).encode())
    return h.hexdigest()[:16]


PROFILE_SQ = os.path.join(ROOT, "profiles", "route_attend_t16k_sq_counters.txt")
SIMDS, CLOCK_GHZ = 1024, 2.4   # MI355X: 256 CUs x 4 SIMDs, peak engine clock


def read_issue(kernel_ms, waves):
    """The route kernel's vector and scalar instruction issue against the
    chip's issue capacity (a wave64 VALU or SALU instruction takes a SIMD's
    issue slot for 4 cycles), from the committed SQ counter summary, or None
    when absent or taken on other kernel source.  The kernel's working set is
    cache resident, so this, not HBM, is what bounds it."""
    if not os.path.exists(PROFILE_SQ):
        return None
    sha, per = None, {}
    for line in open(PROFILE_SQ):
        if "route_source_sha" in line:
            sha = line.split("route_source_sha")[1].split()[0]
        parts = line.lstrip("# ").split()
        if len(parts) >= 2 and parts[0] in ("SQ_INSTS_VALU", "SQ_INSTS_SALU"):
            try:
                per[parts[0]] = float(parts[1])
            except ValueError:   # prose that starts with a counter name
                continue
    if sha != route_source_sha() or len(per) != 2:
        return None
    cap = kernel_ms * 1e-3 * CLOCK_GHZ * 1e9 * SIMDS / 4   # wave64 instructions per SIMD slot
    return {"valu_per_query": per["SQ_INSTS_VALU"], "salu_per_query": per["SQ_INSTS_SALU"],
            "valu_issue_frac": per["SQ_INSTS_VALU"] * waves / cap,
            "salu_issue_frac": per["SQ_INSTS_SALU"] * waves / cap}


def read_traffic(bytes_unit=1024, path=None):
    """HBM bytes per launch of the kernel a committed counter summary covers
    (the fused route kernel by default), or None when absent or taken on
    other kernel source."""
    path = path or PROFILE_COUNTERS
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        line = line.split("#")[0].strip()
        if ":" in line:
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("route_source_sha") != route_source_sha():
        return None
    try:
        f = float(kv["fetch_kib_per_dispatch"]) * float(kv["copy_fetch_factor"])
        w = float(kv["write_kib_per_dispatch"]) * float(kv["copy_write_factor"])
    except (KeyError, ValueError):
        return None
    return (f + w) * bytes_unit


def bytes_per_query(stats, cfg, budget_read=True):
    """Algorithmic bytes of the fused kernel per query from its load counts:
    q row, neighbour key rows, tree rows loaded (left children and cover
    roots; 4d bytes for int32 rows, 2d for int16 rows), key rows loaded by
    the descent, value rows (fp32), the output row, the idx row and the
    count (and the budget it reads)."""
    d = cfg.d
    rows32, rows16, key_rows, C = (stats[..., i].astype(np.int64) for i in range(4))
    n = np.minimum(cfg.window, C)
    b = (d + n * d + rows32 * 4 * d + rows16 * 2 * d + key_rows * d + C * 4 * d + 4 * d
         + 4 * cfg.max_budget + 4 + (4 if budget_read else 0))
    return b


BF16_MFMA_PEAK_TFLOPS = 2500.0


# The dense kernel's P.V split: P and V each as a bf16 head plus a bf16 tail
# (x = hi + lo to within 2^-18 |x|), hi.hi + lo.hi + hi.lo summed in fp32:
# each output within 3 * 2^-18 * max|V| of the fp32 product.
DENSE_PV_REL_BOUND = 3 * 2.0 ** -18
PARITY_ATOL = 1e-4


def dense_summary(w, dense_ms, step_ms, max_abs_v=None):
    """The dense causal baseline's time and its matrix-core roofline: per
    (query, past key) pair 2d int8 ops for the score and, for P.V, three bf16
    products of 2d flops each (heads and tails of P and V), against the bf16
    dense peak (the int8 score work is a thirtieth of it and left out).  The
    precision entry states the split's error bound for this workload's
    values against the routed path's fp32 products."""
    pairs = w.B * w.H * w.T * (w.T + 1) / 2
    bf16_flops = 3 * 2 * w.d * pairs
    achieved = bf16_flops / (dense_ms * 1e-3) / 1e12
    out = {"kernel": "alhr_dense_attend (causal, int8 MFMA scores, P.V as three bf16 MFMA "
                     "products)",
           "ms": dense_ms, "routed_step_speedup": dense_ms / step_ms,
           "roofline": {"bound": "mfma", "achieved": achieved, "peak": BF16_MFMA_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": achieved / BF16_MFMA_PEAK_TFLOPS,
                        "fp32_equivalent_tflops": achieved / 3}}
    if max_abs_v is not None:
        bound = DENSE_PV_REL_BOUND * max_abs_v
        out["precision"] = {
            "pv_abs_error_bound": bound, "max_abs_v": max_abs_v, "parity_atol": PARITY_ATOL,
            "within_parity_atol": bool(bound <= PARITY_ATOL),
            "max_abs_v_for_atol": PARITY_ATOL / DENSE_PV_REL_BOUND,
            "note": "P.V from bf16 heads and tails: each output within 3*2^-18*max|V| of fp32; "
                    "the routed path multiplies in fp32 (no bound on V)"}
    return out


def host_cores():
    """CPUs this process may run on, at most 16 (one GPU's share of a node)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


class pinned_to_one_core:
    """Runs the body on one CPU of this process's set (the calling thread's
    affinity), restoring the set afterwards; yields the CPU used."""

    def __enter__(self):
        self.saved = os.sched_getaffinity(0)
        self.cpu = min(self.saved)
        os.sched_setaffinity(0, {self.cpu})
        return self.cpu

    def __exit__(self, *exc):
        os.sched_setaffinity(0, self.saved)
        return False


def cpu_baseline(w, Q, K, V, W, stride, threads=1):
    """The C oracle on every stride-th query of every (b, h) pair, each pair
    with its own tree build and prefix.  threads > 1 runs whole pairs on that
    many Python threads (the oracle call releases the interpreter lock); the
    oracle itself is unchanged and single-threaded per pair."""
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    cfg = w.config()
    ts = np.arange(0, w.T, stride, dtype=np.int32)
    pairs = [(b, h) for b in range(w.B) for h in range(w.H)]

    def one(bh):
        b, h = bh
        oracle.pair_forward(Q[b, h], K[b, h], V[b, h], W=W, fixed_budget=w.fixed_budget,
                            window=cfg.window, keys_per_class=cfg.keys_per_class,
                            max_budget=cfg.max_budget, scale=cfg.scale, ts=ts)
        return len(ts)

    threads = max(1, min(threads, len(pairs)))
    core = None
    if threads == 1:
        with pinned_to_one_core() as core:
            t0 = time.perf_counter()
            n = sum(one(bh) for bh in pairs)
            dt = time.perf_counter() - t0
    else:
        t0 = time.perf_counter()
        with ThreadPoolExecutor(threads) as ex:
            n = sum(ex.map(one, pairs))
        dt = time.perf_counter() - t0
    return {"value": n / dt, "unit": "queries/s", "cores": threads, "kind": "oracle",
            "sample": "%s: every %d-th query of all %d (b, h) pairs (%d queries), each pair "
                      "with its full tree build and prefix; C oracle, %s, %.1f s"
                      % (w.name, stride, len(pairs), n,
                         ("single-threaded, pinned to CPU %d" % core) if threads == 1
                         else "%d threads over pairs" % threads, dt),
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "process_cpus": len(os.sched_getaffinity(0))}


def bench_splitter(alhr, torch, dev, w, reps=20):
    """Time alhr_split_qk on seeded input rows: batch x T tokens of d_model =
    heads * d int8 features projected to the workload's Q and K."""
    import synth
    dm = w.H * w.d
    X = torch.from_numpy(synth.split_inputs(w.seed, w.B, dm, 0, w.T)).to(dev)
    Wsp = torch.from_numpy(synth.split_weights(w.seed, w.H, w.d, dm)).to(dev)
    scfg = alhr.SplitConfig(batch=w.B, heads=w.H, T=w.T, d=w.d, d_model=dm, shift=6,
                            qclamp=9, kclamp=8)
    Qs, Ks = alhr.alhr_split_qk(scfg, X, Wsp)
    torch.cuda.synchronize()
    # one launch takes about as long as the host needs to submit one, so the
    # launches are captured in a HIP graph (reps per replay) and the events
    # bracket whole replays: the per-launch time is then the GPU's alone
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            alhr.alhr_split_qk(scfg, X, Wsp, Qs, Ks)
    g.replay()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(5)]
    for e in ev:
        e[0].record()
        g.replay()
        e[1].record()
    torch.cuda.synchronize()
    ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev])) / reps
    M, N = w.B * w.T, 2 * w.H * w.d
    ops = 2 * M * N * dm
    nbytes = M * dm + N * dm + M * N
    tops = ops / (ms * 1e-3) / 1e12
    return {"kernel": "k_split (int8 MFMA 32x32x32, 128x256 tiles)",
            "shape": {"tokens": M, "d_model": dm, "outputs": N},
            "ms": ms, "ops_per_launch": ops, "bytes_per_launch": nbytes,
            "roofline": {"bound": "mfma", "achieved": tops, "peak": INT8_MFMA_PEAK_TOPS,
                         "unit": "TOP/s", "frac": tops / INT8_MFMA_PEAK_TOPS},
            "hbm_GBps": nbytes / (ms * 1e-3) / 1e9}


def step_calls(alhr, cfg, q, k, v, wt, nodes, budget, ws, fixed, idx, count, O):
    """One prefill step: the kernels alhr_forward launches, as its two calls
    (tree + budgets in shared launches, then fused route + attend)."""
    alhr.alhr_prepare(cfg, q, k, wt, nodes, budget if wt is not None else None,
                      ws if wt is not None else None)
    alhr.alhr_route_attend(cfg, q, k, v, nodes, budget if wt is not None else None, fixed, idx,
                           count, O)


class TimingEvents:
    """n HIP timing events created with hipEventDisableSystemFence, recorded
    on torch's current stream (the stream the binding launches on).

    A default event ends with a system-scope release: when it completes, the
    GPU writes back and invalidates its caches, so the kernel launched after
    it starts later (about 5 us per event here) and on a cold L2.  These
    events only timestamp the stream; the host reads them after a device
    synchronisation, so they need no fence.  The HIP runtime is the one torch
    has already loaded (same soname), so the stream handles are shared."""

    DISABLE_SYSTEM_FENCE = 0x20000000
    kind = "HIP events without the system-scope fence"

    def __init__(self, torch, n):
        import ctypes
        self._c = ctypes
        hip = ctypes.CDLL("libamdhip64.so.7")
        hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                            ctypes.c_void_p]
        hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self._hip = hip
        self._stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        self._ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            self._check(hip.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE),
                        "hipEventCreateWithFlags")
            self._ev.append(e)

    @staticmethod
    def _check(rc, what):
        if rc != 0:
            raise RuntimeError("%s failed with HIP error %d" % (what, rc))

    def record(self, i):
        self._check(self._hip.hipEventRecord(self._ev[i], self._stream), "hipEventRecord")

    def ms(self, a, b):
        f = self._c.c_float()
        self._check(self._hip.hipEventElapsedTime(self._c.byref(f), self._ev[a], self._ev[b]),
                    "hipEventElapsedTime")
        return f.value

    def close(self):
        for e in self._ev:
            self._hip.hipEventDestroy(e)
        self._ev = []


class TorchEvents:
    """The same interface over torch's default timing events (with the
    system-scope fence), used only when the fence-free events cannot be
    created."""

    kind = "torch default events"

    def __init__(self, torch, n):
        self._ev = [torch.cuda.Event(enable_timing=True) for _ in range(n)]

    def record(self, i):
        self._ev[i].record()

    def ms(self, a, b):
        return self._ev[a].elapsed_time(self._ev[b])

    def close(self):
        self._ev = []


def timing_events(torch, n):
    """n fence-free HIP timing events, or torch's default events (reported
    by their `kind`) when the HIP runtime refuses the flag."""
    try:
        return TimingEvents(torch, n)
    except (OSError, AttributeError, RuntimeError) as e:
        print("bench: fence-free HIP events unavailable (%s); using torch's events" % e,
              file=sys.stderr)
        return TorchEvents(torch, n)


def capture_step(torch, fn):
    """fn's launches captured in a HIP graph (on torch's capture stream, which
    the binding launches on)."""
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    return graph


VALU_PEAK_G = SIMDS * CLOCK_GHZ / 4   # 614.4 G wave64 vector instructions/s
SETTLE_STEPS = 100                     # untimed step replays before the warm-up steps


def route_roofline(kern_ms, queries, bytes_launch, issue, traffic):
    """The fused route + attend kernel against the bound that limits it.

    Its working set (keys, values and the tree of every head, ~70 MiB at
    T = 16384) stays in the caches, so its re-reads of tree, key and value
    rows never reach HBM; what limits it is the vector instruction issue: a
    wave64 VALU instruction holds a SIMD's issue slot for 4 cycles, so the
    chip issues at most 1024 SIMDs x 2.4 GHz / 4 = 614.4 G of them per
    second.  `achieved` = the kernel's VALU instructions per query (committed
    SQ_INSTS_VALU counts for the same source) x queries per launch / the
    launch's event-timed duration.  Beside it: HBM bytes from the committed
    FETCH_SIZE / WRITE_SIZE counts over the same duration against 8 TB/s, and
    the algorithmic bytes touched (row loads counted by the kernel itself),
    which exceed the HBM peak because the re-reads are cache hits.  The counter
    bytes are what leaves L2, part of it served by the MALL: an upper bound on
    the HBM share."""
    sec = kern_ms * 1e-3
    out = {"bound": "alu", "achieved": None, "peak": VALU_PEAK_G,
           "unit": "G wave64 VALU instructions/s", "frac": None, "traffic": traffic,
           "kernel": "k_route (fused route + attend)", "ms_per_launch": kern_ms,
           "queries_per_launch": queries}
    if issue is not None:
        out["achieved"] = issue["valu_per_query"] * queries / sec / 1e9
        out["frac"] = out["achieved"] / VALU_PEAK_G
        out["valu_per_query"] = issue["valu_per_query"]
        out["salu_per_query"] = issue["salu_per_query"]
        out["salu_issue_frac"] = issue["salu_per_query"] * queries / sec / 1e9 / VALU_PEAK_G
    else:
        out["counters"] = "SQ counters absent or taken on other kernel source: no issue figure"
    if traffic is not None:
        gbs = traffic / sec / 1e9
        out["hbm"] = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                      "frac": gbs / HBM_PEAK_GBS, "bytes_per_launch": traffic,
                      "note": "bytes past L2 (FETCH_SIZE + WRITE_SIZE): served by the 256 MB "
                              "MALL or by HBM, so an upper bound on the HBM share"}
    out["bytes_touched"] = {"bytes_per_launch": bytes_launch,
                            "GBps": bytes_launch / sec / 1e9,
                            "note": "algorithmic bytes (rows loaded by the kernel); re-reads "
                                    "are cache hits, so this exceeds what HBM delivers"}
    return out


def bench_prefill(args, torch, dev):
    import learned_tree_routed_amd as alhr
    from synth.workloads import WORKLOADS, host_inputs
    w = WORKLOADS[args.workload]
    if args.budget_override:
        import dataclasses
        w = dataclasses.replace(w, fixed_budget=args.budget_override)
    cfg = w.config()
    Q, K, V, W = host_inputs(w)
    q, k, v = (torch.from_numpy(x).to(dev) for x in (Q, K, V))
    wt = None if W is None else torch.from_numpy(W).to(dev)
    rows = (w.B, w.H, w.T, w.d)
    nodes = torch.empty(rows, dtype=torch.int32, device=dev)
    budget = torch.empty((w.B, w.H, w.T), dtype=torch.int32, device=dev)
    idx = torch.empty((w.B, w.H, w.T, cfg.max_budget), dtype=torch.int32, device=dev)
    count = torch.empty((w.B, w.H, w.T), dtype=torch.int32, device=dev)
    O = torch.empty(rows, dtype=torch.float32, device=dev)
    ws = torch.empty(max(alhr.alhr_workspace_bytes(cfg), 256), dtype=torch.uint8, device=dev)
    fixed = w.fixed_budget

    wb = wt
    bb = budget if wt is not None else None
    wsb = ws if wt is not None else None

    # Untimed work first: the step once eagerly, the routing's load counts
    # for the byte model, the dense baseline and the splitter.  It also brings
    # the GPU to its steady clocks before the timed steps.
    step_calls(alhr, cfg, q, k, v, wt, nodes, budget, ws, fixed, idx, count, O)
    _, _, st = alhr.alhr_route_stats(cfg, q, k, nodes, bb, fixed)
    torch.cuda.synchronize()
    stats = st.cpu().numpy()
    del st
    dense_ms = None
    if w.d >= 32:
        Od = torch.empty_like(O)
        alhr.alhr_dense_attend(cfg, q, k, v, Od)
        dev_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(5)]
        for e in dev_ev:
            e[0].record()
            alhr.alhr_dense_attend(cfg, q, k, v, Od)
            e[1].record()
        torch.cuda.synchronize()
        dense_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in dev_ev]))
        del Od
    # the query/key splitter at this workload's shapes (d_model = heads * d),
    # timed on its own: it precedes the tree path and is not part of a step
    splitter = bench_splitter(alhr, torch, dev, w)

    # The timed steps: each one is the two calls, the preparation (tree +
    # budgets, alhr_prepare) and the fused route + attend (alhr_route_attend),
    # launched directly, with a fence-free HIP timing event on the launch
    # stream before and after the route call, so the route kernel's duration
    # is measured in the timed region itself; the span from one route call's
    # end to the next one's start is the preparation with its launch gaps.
    # A step takes about half a millisecond of GPU time and its three launches
    # a few tens of microseconds of host time, so the host stays ahead and the
    # kernels run back to back (replaying each call as a HIP graph instead
    # added about 8 microseconds per graph on this platform; torch's default
    # events, three per step, added about 10 microseconds per step through
    # their cache write-back and invalidation).
    def prep():
        alhr.alhr_prepare(cfg, q, k, wb, nodes, bb, wsb)

    def route():
        alhr.alhr_route_attend(cfg, q, k, v, nodes, bb, fixed, idx, count, O)

    # untimed settle phase: the GPU reaches its steady clocks after a few tens
    # of milliseconds of this kernel (with 5 steps only, the timed route
    # launches ran 5% slower), then the W warm-up steps
    for _ in range(SETTLE_STEPS + args.warmup):
        prep()
        route()
    events = timing_events(torch, 2 * args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        prep()
        events.record(2 * i)
        route()
        events.record(2 * i + 1)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    kern = {"route_attend_ms": float(np.mean([events.ms(2 * i, 2 * i + 1)
                                              for i in range(args.steps)])),
            "prepare_and_gaps_ms": (float(np.mean([events.ms(2 * i - 1, 2 * i)
                                                   for i in range(1, args.steps)]))
                                    if args.steps > 1 else None),
            "events": events.kind}
    events.close()

    bpl = int(bytes_per_query(stats, cfg, wt is not None).sum())
    counted = args.workload == "t16k" and not args.budget_override
    traffic = read_traffic() if counted else None
    queries = w.B * w.H * w.T
    issue = read_issue(kern["route_attend_ms"], queries) if counted else None
    cnt = count.cpu().numpy()
    bud = budget.cpu().numpy() if wt is not None else np.full_like(cnt, fixed)
    out = {
        "metric": "routed queries/sec (build+route+attend) at T=%d; %% of HBM peak" % w.T,
        "value": queries / (ms_step * 1e-3),
        "unit": "queries/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step, "settle_steps": SETTLE_STEPS,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "i8/i32 routing, f32 attention",
        "data": "synthetic (clustered int8 keys, noisy copied queries, seeded)",
        "config": {"workload": w.name, "batch": w.B, "heads": w.H, "T": w.T, "d": w.d,
                   "window": cfg.window, "max_budget": cfg.max_budget,
                   "budget": ("fixed %d" % fixed) if fixed else "int8 predictor, 32 classes x 3",
                   "queries_per_step": queries,
                   "launch": "per step: alhr_prepare (build + predict), then "
                             "alhr_route_attend, launched back to back"},
        "roofline": route_roofline(kern["route_attend_ms"], queries, bpl, issue, traffic),
        "kernels_ms": kern,
        "dense_baseline": None if dense_ms is None else dense_summary(
            w, dense_ms, ms_step, float(np.abs(V).max())),
        "splitter": splitter,
        "diagnostics": {"mean_budget": float(bud.mean()), "mean_keys_per_query": float(cnt.mean()),
                        "budget_histogram": {int(v): int(c) for v, c in
                                             zip(*np.unique(bud, return_counts=True))},
                        "mean_tree_rows_loaded_int32": float(stats[..., 0].mean()),
                        "mean_tree_rows_loaded_int16": float(stats[..., 1].mean()),
                        "mean_key_rows_loaded": float(stats[..., 2].mean()),
                        "bytes_per_query": bpl / queries,
                        "compression_T_over_keys": float(w.T / cnt.mean()),
                        "compression_causal_over_keys": float((w.T + 1) / 2 / cnt.mean())},
    }
    return out, (w, Q, K, V, W)


def decode_measure(torch, dev, steps, warmup, with_cpu=True):
    """The decode workload: 64 sequences x 16 heads, a cache of 2^17 - 128 keys
    (d = 128, 144 GiB of keys, values and tree, generated on the device), then
    128 tokens, each one launch of alhr_append_decode (append the key and
    value, add the key to its ancestors and to the running sum, then predict,
    route and attend the token's query for every pair).  The 128 launches are
    one HIP graph; each timed replay starts from the same cache (rebuilt,
    untimed)."""
    import learned_tree_routed_amd as alhr
    from synth import device as sd
    from synth.workloads import WORKLOADS
    w = WORKLOADS["decode"]
    cfg = w.config()
    B, H, T, d, n0, S = w.B, w.H, w.T, w.d, w.n0, w.steps
    K = torch.zeros((B, H, T, d), dtype=torch.int8, device=dev)
    V = torch.zeros((B, H, T, d), dtype=torch.float32, device=dev)
    nodes = torch.empty((B, H, T, d), dtype=torch.int32, device=dev)
    sd.keys_(K, w.seed, 0, n0)
    sd.values_(V, w.seed, 0, n0)
    Wd = sd.weights_(torch.empty((32, 2 * d), dtype=torch.int8, device=dev), w.seed)
    kn = sd.keys_(torch.empty((B, H, S, d), dtype=torch.int8, device=dev), w.seed, n0)
    vn = sd.values_(torch.empty((B, H, S, d), dtype=torch.float32, device=dev), w.seed, n0)
    qn = sd.queries_(torch.empty((B, H, S, d), dtype=torch.int8, device=dev), w.seed, n0)
    ks = [kn[:, :, s].contiguous() for s in range(S)]
    vs = [vn[:, :, s].contiguous() for s in range(S)]
    qs = [qn[:, :, s].contiguous() for s in range(S)]
    idx = torch.empty((B, H, cfg.max_budget), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, H), dtype=torch.int32, device=dev)
    O = torch.empty((B, H, d), dtype=torch.float32, device=dev)
    bud = torch.empty((B, H), dtype=torch.int32, device=dev)
    prefix = torch.empty((B, H, d), dtype=torch.int32, device=dev)

    def reset():
        # untimed: drop the appended rows and rebuild the cache of n0 keys
        K[:, :, n0:].zero_()
        V[:, :, n0:].zero_()
        alhr.alhr_build_tree(cfg, K, nodes)
        alhr.alhr_prefix_from_tree(cfg, n0, K, nodes, prefix)

    def loop():
        for s in range(S):
            alhr.alhr_append_decode(cfg, n0 + s, ks[s], vs[s], qs[s], K, V, nodes, prefix, Wd, 0,
                                    bud, idx, cnt, O)

    reset()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    loop()
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3
    graph = torch.cuda.CUDAGraph()
    reset()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        loop()
    for _ in range(warmup):
        reset()
        graph.replay()
    times = []
    for _ in range(steps):
        reset()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev[0].record()
        graph.replay()
        ev[1].record()
        torch.cuda.synchronize()
        times.append(((time.perf_counter() - t0) * 1e3, ev[0].elapsed_time(ev[1])))
    ms = float(np.mean([t[0] for t in times]))
    ev_ms = float(np.mean([t[1] for t in times]))
    queries = B * H * S
    roof, picks = decode_roofline(alhr, torch, dev, w, cfg, K, nodes, qn, Wd, bud, cnt, ev_ms)
    out = {"metric": "routed queries/sec (append+route+attend), decode at T=2^17",
           "value": queries / (ms * 1e-3), "unit": "queries/s", "ms_per_step": ms,
           "steps": steps, "warmup": warmup,
           "config": {"workload": "decode", "sequences": B, "heads": H, "T": T, "d": d,
                      "prefilled": n0, "tokens_per_step": S, "queries_per_step": queries,
                      "launch": "HIP graph of 128 alhr_append_decode launches (one per token)"},
           "roofline": roof,
           "diagnostics": {"mean_keys_last_step": float(cnt.float().mean().item()),
                           "event_ms_per_step": ev_ms, "eager_ms_per_step": eager_ms}}
    if with_cpu:
        out["cpu_baseline"] = decode_cpu_baseline(torch, w, cfg, K, V, qn, Wd, picks)
    del K, V, nodes, kn, vn, qn
    torch.cuda.empty_cache()
    return out


def decode_cpu_baseline(torch, w, cfg, K, V, qn, Wd, picks):
    """The oracle replaying the 128 decode steps (append, predictor, route,
    attend) of sampled (sequence, head) pairs on one pinned host core.  Each
    pair's prefilled cache and tree are set up untimed, as on the GPU; the
    key, value and query rows are copied from the device buffers the GPU run
    used (drawn by the seeded generator)."""
    import oracle
    n0, S, T, d = w.n0, w.steps, w.T, w.d
    W = Wd.cpu().numpy()
    total, nq = 0.0, 0
    with pinned_to_one_core() as core:
        for pidx in picks:
            b, h = divmod(int(pidx), w.H)
            Kp = K[b, h].cpu().numpy()
            Vp = V[b, h].cpu().numpy()
            Qp = qn[b, h].cpu().numpy()
            Kc = np.zeros_like(Kp)
            Kc[:n0] = Kp[:n0]
            Vc = np.zeros_like(Vp)
            Vc[:n0] = Vp[:n0]
            tree = oracle.build_tree(Kc)
            pre = Kc.astype(np.int64).sum(axis=0)
            t0 = time.perf_counter()
            for s in range(S):
                p = n0 + s
                oracle.append(p, Kp[p], Vp[p], Kc, Vc, tree, pre)
                bt, _ = oracle.budget(Qp[s], pre, W, cfg.keys_per_class, cfg.max_budget)
                ix, _, c, _ = oracle.route(p, bt, Qp[s], Kc, tree, cfg.window, cfg.max_budget)
                oracle.attend(ix[:c], Qp[s], Kc, Vc, cfg.scale)
            total += time.perf_counter() - t0
            nq += S
            del Kp, Vp, Kc, Vc, tree
    return {"value": nq / total, "unit": "queries/s", "cores": 1, "kind": "oracle",
            "sample": "decode: %d sampled (sequence, head) pairs x %d steps (append + predictor "
                      "+ route + attend), prefilled cache built untimed; C oracle, single-"
                      "threaded, pinned to CPU %d, %.2f s" % (len(picks), S, core, total),
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "process_cpus": len(os.sched_getaffinity(0))}


def bench_decode(args, torch, dev):
    d = decode_measure(torch, dev, args.steps, args.warmup, with_cpu=not args.no_cpu_baseline)
    out = {"metric": d["metric"], "value": d["value"], "unit": d["unit"],
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": d["ms_per_step"],
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "i8/i32 routing, f32 attention",
           "data": "synthetic (device-generated clustered keys, seeded)",
           "config": d["config"], "roofline": d["roofline"], "diagnostics": d["diagnostics"]}
    if "cpu_baseline" in d:
        out["cpu_baseline"] = d["cpu_baseline"]
    return out, None


def decode_roofline(alhr, torch, dev, w, cfg, K, nodes, qn, Wd, bud, cnt, event_ms_loop,
                    npairs=8):
    """Algorithmic bytes of k_decode (append + route + attend) per token step
    over its event-timed duration.  The per-query load counts come from
    alhr_route_stats on sampled (sequence, head) pairs of the final cache, with
    the decode queries at their positions: a query at position p reads only
    subtrees of [0, p] and S[p], which later appends leave unchanged, so the
    counts are those of the decode launches.  Append bytes per pair and token:
    the key and value rows written, each ancestor row and the running key sum
    read and written; the predictor reads the updated sum and, once per
    step, the shared weights."""
    B, H, T, d, n0, S = w.B, w.H, w.T, w.d, w.n0, w.steps
    cfg1 = w.config(batch=1, heads=1)
    l16 = alhr.alhr_tree_int16_levels(cfg1)
    L = T.bit_length() - 1
    rng = np.random.default_rng(w.seed)
    picks = rng.choice(B * H, size=min(npairs, B * H), replace=False)
    per_query = []
    for pidx in picks:
        b, h = divmod(int(pidx), H)
        Kp = K[b:b + 1, h:h + 1].contiguous()
        Np = nodes[b:b + 1, h:h + 1].contiguous()
        Qp = torch.zeros((1, 1, T, d), dtype=torch.int8, device=dev)
        Qp[0, 0, n0:n0 + S] = qn[b, h]
        bp = alhr.alhr_predict_budget(cfg1, Qp, Kp, Wd)
        _, cp, st = alhr.alhr_route_stats(cfg1, Qp, Kp, Np, bp, 0)
        torch.cuda.synchronize()
        # the last decode step of this pair must match what the decode launch chose
        last = n0 + S - 1
        assert int(bp[0, 0, last]) == int(bud[b, h]) and int(cp[0, 0, last]) == int(cnt[b, h]), \
            "route_stats disagrees with the decode launch at pair (%d, %d)" % (b, h)
        sel = st[0, 0, n0:n0 + S].cpu().numpy()
        per_query.append(bytes_per_query(sel, cfg, budget_read=True))
        del Kp, Np, Qp
    route_b = float(np.mean(np.concatenate(per_query)))
    anc = sum((2 * d if lvl <= l16 else 4 * d) for lvl in range(1, L + 1))
    append_b = d + 4 * d + 2 * anc + 2 * 4 * d
    # the predictor weights are shared by every query of the step: counted once
    bytes_token = (route_b + append_b) * B * H + cfg.n_classes * 2 * d
    ms_token = event_ms_loop / S
    achieved = bytes_token / (ms_token * 1e-3) / 1e9
    traffic = read_traffic(path=PROFILE_DECODE_COUNTERS)
    out = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
           "kernel": "k_decode (append + route + attend, one launch per token)",
           "bytes_per_launch": bytes_token, "ms_per_launch": ms_token,
           "sample": "load counts of the %d decode queries of %d sampled pairs "
                     "(alhr_route_stats on the final cache)" % (S * len(picks), len(picks))}
    if traffic is not None:
        gbs = traffic / (ms_token * 1e-3) / 1e9
        out["hbm_counted"] = {"achieved": gbs, "frac": gbs / HBM_PEAK_GBS,
                              "note": "FETCH_SIZE + WRITE_SIZE per launch (committed counters) "
                                      "over the same duration"}
    return out, picks


def bench_sweep(args, torch, dev):
    """Length sweep (T = 2^10 .. 2^17, B1 H8 d64, predictor): time per step and
    per fused launch, the per-query load counts, the device footprint, and a
    least-squares exponent of time vs T."""
    import learned_tree_routed_amd as alhr
    from synth import device as sd
    from synth.workloads import Workload
    lines, Ts, ms_all = [], [], []
    for L in range(10, 18):
        T = 1 << L
        w = Workload("sweep", 4, 1, 8, T, 64, "clustered")
        cfg = w.config()
        shape = (w.B, w.H, T, w.d)
        K = sd.keys_(torch.empty(shape, dtype=torch.int8, device=dev), w.seed)
        Q = sd.queries_(torch.empty(shape, dtype=torch.int8, device=dev), w.seed)
        V = sd.values_(torch.empty(shape, dtype=torch.float32, device=dev), w.seed)
        Wt = sd.weights_(torch.empty((32, 128), dtype=torch.int8, device=dev), w.seed)
        nodes = torch.empty(shape, dtype=torch.int32, device=dev)
        bud = torch.empty((1, 8, T), dtype=torch.int32, device=dev)
        idx = torch.empty((1, 8, T, cfg.max_budget), dtype=torch.int32, device=dev)
        cnt = torch.empty((1, 8, T), dtype=torch.int32, device=dev)
        O = torch.empty(shape, dtype=torch.float32, device=dev)
        ws = torch.empty(max(alhr.alhr_workspace_bytes(cfg), 256), dtype=torch.uint8, device=dev)

        evs = timing_events(torch, 2 * args.steps)

        def step(i):
            alhr.alhr_prepare(cfg, Q, K, Wt, nodes, bud, ws)
            if i is not None:
                evs.record(2 * i)
            alhr.alhr_route_attend(cfg, Q, K, V, nodes, bud, 0, idx, cnt, O)
            if i is not None:
                evs.record(2 * i + 1)
        for _ in range(2):
            step(None)
        torch.cuda.synchronize()
        for i in range(args.steps):
            step(i)
        torch.cuda.synchronize()
        kms = float(np.mean([evs.ms(2 * i, 2 * i + 1) for i in range(args.steps)]))
        evs.close()
        # step time from graph replays of the same calls (at the short lengths
        # a step takes about as long as the host needs to issue its launches)
        graph = capture_step(torch, lambda: step_calls(alhr, cfg, Q, K, V, Wt, nodes, bud, ws, 0,
                                                       idx, cnt, O))
        for _ in range(max(1, args.warmup)):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / args.steps
        del graph
        _, _, st = alhr.alhr_route_stats(cfg, Q, K, nodes, bud, 0)
        stats = st.cpu().numpy()
        bpl = int(bytes_per_query(stats, cfg).sum())
        state = K.numel() + 4 * V.numel() + 4 * nodes.numel()
        alhr.alhr_dense_attend(cfg, Q, K, V, O)
        de = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(3)]
        for e in de:
            e[0].record()
            alhr.alhr_dense_attend(cfg, Q, K, V, O)
            e[1].record()
        torch.cuda.synchronize()
        dense_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in de]))
        q = w.B * w.H * T
        lines.append({"sweep_T": T, "queries": q, "ms_per_step": ms, "route_attend_ms": kms,
                      "routed_qps": q / (ms * 1e-3),
                      "route_attend_GBps": bpl / (kms * 1e-3) / 1e9,
                      "mean_keys": float(cnt.float().mean().item()),
                      "mean_tree_rows": float(stats[..., 0].mean() + stats[..., 1].mean()),
                      "cache_bytes_K_V_tree": state,
                      "dense_ms": dense_ms, "dense_over_routed_step": dense_ms / ms})
        Ts.append(T)
        ms_all.append(ms)
        del K, Q, V, nodes, idx, O
        torch.cuda.empty_cache()
    x = np.log(np.array(Ts, dtype=np.float64))
    y = np.log(np.array(ms_all))
    alpha = float(np.polyfit(x, y, 1)[0])
    alpha_dense = float(np.polyfit(x, np.log(np.array([l["dense_ms"] for l in lines])), 1)[0])
    per_q = np.array(ms_all) / np.array(Ts)
    beta = float(np.polyfit(np.log2(np.array(Ts, dtype=np.float64)), per_q / per_q[0], 1)[0])
    return lines, {"sweep_fit": {"exponent_time_vs_T": alpha,
                                 "exponent_dense_time_vs_T": alpha_dense,
                                 "per_query_time_growth_per_doubling": beta,
                                 "T_range": [Ts[0], Ts[-1]]}}


def bench_quality(args, torch, dev):
    """Routing quality on the synthetic recall task: how often the selected
    set holds the key the query was copied from, and how much of the dense
    top-16 (by q . k, the label the README's phase 2 distils) it holds."""
    import dataclasses
    import learned_tree_routed_amd as alhr
    import synth
    from synth.workloads import WORKLOADS, host_inputs
    out = []
    rng = np.random.default_rng(0)
    for name in ("t1k", "t16k"):
        base = WORKLOADS[name]
        Q, K, V, W = host_inputs(base)
        q, k = (torch.from_numpy(x).to(dev) for x in (Q, K))
        src = synth.query_sources(base.seed, base.B, base.H, 0, base.T)
        cfg = base.config()
        nodes = alhr.alhr_build_tree(cfg, k)
        wt = torch.from_numpy(W).to(dev)
        pred = alhr.alhr_predict_budget(cfg, q, k, wt)
        samples = [(int(rng.integers(base.B)), int(rng.integers(base.H)),
                    int(rng.integers(64, base.T))) for _ in range(256)]
        top16 = {}
        for (b, h, t) in samples:
            sc = K[b, h, :t + 1].astype(np.int64) @ Q[b, h, t].astype(np.int64)
            order = np.lexsort((np.arange(t + 1), -sc))
            top16[(b, h, t)] = set(order[:16].tolist())
        for budget in (8, 16, 30, 48, 64, 96, 0):
            bud = pred if budget == 0 else None
            idx, cnt = alhr.alhr_route(cfg, q, k, nodes, bud, budget)
            I = idx.cpu().numpy()
            C = cnt.cpu().numpy()
            t = np.arange(base.T)
            hit = (I == src[..., None]).any(axis=-1)[..., 1:]
            d16 = np.mean([len(top16[x] & set(I[x][:C[x]].tolist())) / 16 for x in samples])
            out.append({"quality_workload": name, "budget": budget or "predictor",
                        "mean_keys": float(C.mean()),
                        "source_key_recall": float(hit.mean()),
                        "dense_top16_recall_sampled": float(d16),
                        "window_only_source_recall": float(
                            ((t[None, None, 1:] - src[..., 1:]) < cfg.window).mean())})
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up steps (default: 20 for prefill workloads, 1 for "
                         "decode); untimed auxiliary measurements run before them")
    ap.add_argument("--workload", default="t16k", choices=["tiny", "t1k", "t4k", "t16k", "decode"])
    ap.add_argument("--budget-override", type=int, default=0,
                    help="fixed budget for every query instead of the predictor (context runs)")
    ap.add_argument("--cpu-stride", type=int, default=1,
                    help="oracle baseline routes every k-th query of every pair")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true",
                    help="leave out the decode sub-measurement of the default (t16k) run")
    ap.add_argument("--decode-steps", type=int, default=3,
                    help="timed 128-token loops of the decode sub-measurement")
    ap.add_argument("--sweep", action="store_true",
                    help="length sweep T = 2^10..2^17 with an exponent fit (JSON line per T)")
    ap.add_argument("--quality", action="store_true",
                    help="routing-quality diagnostics: source-key and dense top-16 recall")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB read + 1 GiB write elementwise kernel (x5), the "
                         "reference for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE")
    args = ap.parse_args()
    if args.warmup is None:
        args.warmup = 1 if args.workload == "decode" else 20
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build measures one GPU; the ALHR path shards by (batch, head) "
              "pair with no exchange, and no multi-GPU run is part of it (--gpus %d requested)"
              % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = (1 << 30) // 4
        x = torch.ones(n, dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        for _ in range(5):
            torch.neg(x, out=y)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration": {"kernel": "elementwise neg, fp32",
                                               "read_bytes": 4 * n, "write_bytes": 4 * n,
                                               "dispatches": 5}}), flush=True)
        return
    if args.sweep:
        lines, fit = bench_sweep(args, torch, dev)
        for line in lines:
            print(json.dumps(line), flush=True)
        print(json.dumps(fit), flush=True)
        return
    if args.quality:
        for line in bench_quality(args, torch, dev):
            print(json.dumps(line), flush=True)
        return
    if args.workload == "decode":
        out, inputs = bench_decode(args, torch, dev)
    else:
        out, inputs = bench_prefill(args, torch, dev)
    if inputs is not None and not args.no_cpu_baseline:
        w, Q, K, V, W = inputs
        out["cpu_baseline"] = cpu_baseline(w, Q, K, V, W, args.cpu_stride)
        cores = host_cores()
        if cores > 1:
            out["cpu_baseline_all_cores"] = cpu_baseline(w, Q, K, V, W, args.cpu_stride, cores)
    if args.workload == "t16k" and not args.budget_override and not args.no_decode:
        # the decode workload (the HBM-bound case) in the same line, after the
        # timed prefill steps
        torch.cuda.empty_cache()
        try:
            out["decode"] = decode_measure(torch, dev, args.decode_steps, 1,
                                           with_cpu=not args.no_cpu_baseline)
        except RuntimeError as e:   # e.g. less free device memory than its 144 GiB cache
            # the headline line is still printed; the decode entry says why it is missing
            out["decode"] = {"error": "%s: %s" % (type(e).__name__, str(e)[:300])}
            torch.cuda.empty_cache()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

"""Benchmark: fused indexer scoring + exact top-2048 on one MI355X.

One step = one complete operator call over one batch of seeded synthetic
input already resident in HBM: for prefill the threshold sampler, the fused
main kernel and the exact repair (idx_topk_prefill); for paged decode the
split scoring kernel and the per-sequence exact selection
(idx_topk_decode_paged).  Throughput counts
the scoring the valid ranges require (Fusing Indexer Scoring and Exact Top-k
page, "5.1 Version trajectory" equation): pairs = sum over rows of the range
length, 2*64*128 FLOP per pair.

The timed calls go through the *_debug entry points with nothing set but a
pair of HIP events recorded on the call's stream right around the dominant
kernel; kernels and arguments are otherwise those of the plain entry points.

Prints ONE JSON line.  The roofline object is for the dominant kernel:
k_prefill_pair (bound by FP8 MFMA) for prefill, k_decode_score (bound by
HBM) for decode.  For prefill it also carries the main kernel's mean shader
clock, measured inside the kernel (shader-clock cycles over constant-rate
wall-clock ticks of every wave), and the fraction of the peak at that clock;
beside it, the control of "5.2 Math-only control" (the main
kernel's loads, MFMAs and scores with no sampling, filtering, selection or
repair) gives the selection time the complete operator leaves exposed.  The
short-context cases (prefill smoke, paged decode) are also timed cold: a
512 MiB buffer is written and read back between calls, so that the 256 MB
Infinity Cache holds none of the inputs and no dirty line of its own.
"""
from __future__ import annotations

import argparse
import ctypes
import glob
import hashlib
import json
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

FLOP_PER_PAIR = 2 * 64 * 128
FP8_DENSE_PEAK_TFLOPS = 5000.0  # MI355X dense FP8 MFMA
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
METRIC = "fused score+top-2048 Gqk-pairs/s and % FP8 MFMA peak at 128K ctx, 1 MI355X"
PREFILL = ["long_prefill", "prefill_chunk", "prefill_smoke", "adversarial"]
COLD = ["prefill_smoke", "paged_decode"]  # short-context cases: also timed with cold caches
DECODE = ["paged_decode"]
SCAN = ["bf16_scan"]
SCAN_METRIC = "BF16 stream scan + exact top-2048, GB/s of keys, 32 streams x 262144 keys, 1 MI355X"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


NOMINAL_CLOCK_GHZ = 2.4  # the clock the FP8 peak is quoted at


def wall_clock_khz() -> int:
    """Rate of the constant wall clock the kernels read (hipDeviceAttributeWallClockRate)."""
    hip = ctypes.CDLL("libamdhip64.so")
    v = ctypes.c_int(0)
    if hip.hipDeviceGetAttribute(ctypes.byref(v), 10017, torch.cuda.current_device()) != 0 or v.value <= 0:
        raise RuntimeError("hipDeviceGetAttribute(WallClockRate) failed")
    return v.value


class CacheFlush:
    """Writes a 512 MiB buffer, then reads it back: afterwards the 256 MB
    Infinity Cache and the L2s hold none of a call's inputs, and no dirty
    line of the flush is left to be written back during the timed call."""

    def __init__(self):
        self.buf = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        self.acc = torch.zeros((), dtype=torch.int64, device="cuda")
        self.n = 0

    def __call__(self):
        self.n += 1
        self.buf.fill_(self.n & 0xFF)
        self.acc += self.buf.view(torch.int64).sum()


def timed_cold(step, steps: int):
    """Calls after a cache flush: (mean call ms, mean dominant-kernel ms).
    Each call's time runs from an event recorded after its flush to one
    recorded after the call, with no event inside the call (so it includes
    the dispatch of the call's first kernel); the dominant kernel's time
    comes from a second set of flushed calls whose launches record events."""
    flush = CacheFlush()

    def pairs():
        return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]

    calls, kern = pairs(), pairs()
    for e0, e1 in kern:  # torch creates the HIP events on first record; the library records them again
        e0.record()
        e1.record()
    for i in range(steps):
        flush()
        calls[i][0].record()
        step(None, 1)
        calls[i][1].record()
    for i in range(steps):
        flush()
        step([kern[i]], 1)
    torch.cuda.synchronize()
    call_ms = [a.elapsed_time(b) for a, b in calls]
    kern_ms = [a.elapsed_time(b) for a, b in kern]
    return float(np.mean(call_ms)), float(np.mean(kern_ms))


def tensor(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()


def oracle_threads() -> int:
    threads = len(os.sched_getaffinity(0))
    if os.environ.get("OMP_NUM_THREADS"):
        threads = min(threads, int(os.environ["OMP_NUM_THREADS"]))
    return threads


def cpu_baseline_prefill(case, seconds: float, chunk: int = 64):
    """The oracle as it stands, on a bounded sample of full rows: chunks of
    rows from a seeded permutation until `seconds` of work have been done."""
    import oracle
    order = np.random.default_rng(0).permutation(case.Q).astype(np.int32)
    threads = oracle_threads()
    done, pairs, dt = 0, 0, 0.0
    while done < case.Q and dt < seconds:
        rows = np.sort(order[done:done + chunk])
        t0 = time.perf_counter()
        oracle.prefill_case(case, rows=rows, want_scores=False, nthreads=threads)
        dt += time.perf_counter() - t0
        pairs += int((case.row_end[rows].astype(np.int64) - case.row_start[rows]).sum())
        done += len(rows)
    return {"value": pairs / dt / 1e9, "unit": "Gqk-pairs/s", "cores": threads, "kind": "oracle",
            "sample": "%d of %d rows of %s (seeded random full rows, fp64 exact scoring + full "
                      "sort per row), %.1f s" % (done, case.Q, case.name, dt)}


def cpu_baseline_decode(case, seconds: float):
    """The oracle on the whole decode batch, repeated until `seconds`."""
    import oracle
    threads = oracle_threads()
    reps, dt = 0, 0.0
    while reps == 0 or dt < seconds:
        t0 = time.perf_counter()
        oracle.decode_case(case, want_scores=False, nthreads=threads)
        dt += time.perf_counter() - t0
        reps += 1
    return {"value": case.pairs * reps / dt / 1e9, "unit": "Gqk-pairs/s", "cores": threads,
            "kind": "oracle",
            "sample": "the whole %s batch (%d sequences, %d keys) x %d, fp64 exact scoring + full "
                      "sort per sequence, %.1f s" % (case.name, case.B, case.pairs, reps, dt)}


KERNEL_SOURCE = {"k_prefill_pair": "idx_prefill.hip", "k_decode_score": "idx_decode.hip",
                 "k_scan_bf16": "idx_scan.hip"}


def source_digest(kernel: str) -> str:
    """sha256 over the source file that defines `kernel`, every header of the
    library, the public header and the build flags: the stored counters stay
    valid while none of these change."""
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "scoring_exact_top_amd")
    files = ([os.path.join(pkg, "csrc", KERNEL_SOURCE[kernel])] +
             sorted(glob.glob(os.path.join(pkg, "csrc", "*.hpp"))) +
             [os.path.join(ROOT, "include", "idx_topk.h"), os.path.join(pkg, "build.py")])
    for f in files:
        h.update(os.path.relpath(f, ROOT).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def stored_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed counter summary,
    or None when there is none for this workload or it covers other sources."""
    path = os.path.join(ROOT, "profiles", "%s_%s_hbm_traffic.md" % (kernel, workload))
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_b = re.search(r"^traffic_bytes_per_launch\s*=\s*(\d+)", text, re.M)
    m_h = re.search(r"^source_sha256\s*=\s*([0-9a-f]{64})", text, re.M)
    if not (m_b and m_h) or m_h.group(1) != source_digest(kernel):
        return None
    return int(m_b.group(1))


def calibrate_copy(mib: int):
    """A plain device-to-device copy of `mib` MiB, the reference for scaling
    the FETCH_SIZE / WRITE_SIZE counters."""
    x = torch.ones(mib << 18, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    y.copy_(x)
    torch.cuda.synchronize()
    log("copied %d MiB" % mib)


def timed(step, n_calls: int, steps: int, warmup: int):
    """Run `warmup` untimed steps, then `steps` timed ones bracketed by
    synchronisation, without any event inside the steps (ms per step); then
    `steps` more in which step(evs, reps) has call j launch its dominant
    kernel `reps` times back to back with evs[j] recorded by the first and
    the last launch (reps is chosen so that these spans last about 2 ms: one
    dispatch's latency does not then dominate a small kernel's duration).
    Returns (ms per step, mean dominant-kernel ms per launch, min)."""
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(n_calls)] for _ in range(steps)]
    for step_evs in evs:  # torch creates the HIP events on first record
        for e0, e1 in step_evs:
            e0.record()
            e1.record()
    for _ in range(warmup):
        step(None, 1)
    torch.cuda.synchronize()
    t_begin = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_begin.record()
    for s in range(steps):
        step(None, 1)
    t_end.record()
    torch.cuda.synchronize()
    ms_per_step = t_begin.elapsed_time(t_end) / steps
    reps = int(min(50, max(1, round(2.0 / (ms_per_step / n_calls)))))
    for s in range(steps):
        step(evs[s], reps)
    torch.cuda.synchronize()
    per_step = [sum(e0.elapsed_time(e1) for e0, e1 in step_evs) / reps for step_evs in evs]
    return ms_per_step, float(np.mean(per_step)) / n_calls, min(per_step) / n_calls


def with_graph(args, lib, step):
    """With --graph: the plain step, step(None, 1), recorded once into a HIP
    graph (idx_topk_graph_*) and replayed; the event-timed steps stay eager
    (their events are recorded by the launches themselves)."""
    if not args.graph:
        return step
    step(None, 1)
    torch.cuda.synchronize()
    g = lib.capture(lambda: step(None, 1))

    def gstep(step_evs, reps):
        if step_evs is None and reps == 1:
            g.launch()
        else:
            step(step_evs, reps)
    gstep.graph = g
    return gstep


def result(args, value, ms_per_step, config, roofline, dtype):
    return {"metric": METRIC, "value": value, "unit": "Gqk-pairs/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
            "data": "synthetic (seeded Gaussian, e4m3 with amax/448 scales)", "config": config,
            "roofline": roofline}


def bench_prefill(args, lib):
    made = synth.WORKLOADS[args.workload](0)
    cases = made if isinstance(made, list) else [made]
    pairs = sum(c.pairs for c in cases)
    devs = [{k: tensor(getattr(c, k)) for k in
             ("q8", "q_scale", "k8", "k_scale", "w", "row_start", "row_end")} for c in cases]
    outs = [torch.empty((c.Q, c.K), dtype=torch.int32, device="cuda") for c in cases]
    wss = [lib.alloc_workspace(lib.prefill_workspace_bytes(c.Q, c.N, c.K), "cuda") for c in cases]
    n_calls = len(cases)

    def step(step_evs, reps):
        for j, (c, d) in enumerate(zip(cases, devs)):
            lib.prefill_debug(d["q8"], d["q_scale"], d["k8"], d["k_scale"], d["w"], d["row_start"],
                              d["row_end"], c.K, out=outs[j], workspace=wss[j],
                              main_events=None if step_evs is None else step_evs[j], main_reps=reps)

    ms_per_step, main_avg, main_min = timed(with_graph(args, lib, step), n_calls, args.steps, args.warmup)
    log("workload", args.workload, "pairs", pairs, "ms/step %.4f" % ms_per_step,
        "main kernel ms/launch %.4f (min %.4f)" % (main_avg, main_min))
    subcalls = []
    for c, ws in zip(cases, wss):
        st = lib.read_stats(ws)
        log("  ", c.name, st)
        subcalls.append(dict(name=c.name, keys=c.N, pairs=c.pairs, **st))

    # mean shader clock of the main kernel, read inside it (untimed pass)
    clk = torch.zeros(2, dtype=torch.int64, device="cuda")
    for j, (c, d) in enumerate(zip(cases, devs)):
        for _ in range(args.steps):
            lib.prefill_debug(d["q8"], d["q_scale"], d["k8"], d["k_scale"], d["w"], d["row_start"],
                              d["row_end"], c.K, out=outs[j], workspace=wss[j], clock_out=clk)
    torch.cuda.synchronize()
    cycles, ticks = (int(x) for x in clk.cpu().tolist())
    clock_ghz = cycles / ticks * wall_clock_khz() * 1e-6 if ticks > 0 else None
    log("main kernel mean shader clock %.3f GHz" % clock_ghz if clock_ghz else "no clock reading")

    # the Math-only control of the main kernel (no sampling, filter, selection or repair)
    def step_control(step_evs, reps):
        for j, (c, d) in enumerate(zip(cases, devs)):
            lib.prefill_debug(d["q8"], d["q_scale"], d["k8"], d["k_scale"], d["w"], d["row_start"],
                              d["row_end"], c.K, out=outs[j], workspace=wss[j], math_only=True,
                              main_events=None if step_evs is None else step_evs[j], main_reps=reps)

    ms_control, control_avg, _ = timed(step_control, n_calls, args.steps, args.warmup)
    log("control (Math-only) ms/step %.4f, exposed selection %.2f%%"
        % (ms_control, 100.0 * (ms_per_step - ms_control) / ms_per_step))
    achieved = FLOP_PER_PAIR * (pairs / n_calls) / (main_avg * 1e-3) / 1e12
    config = {"workload": cases[0].name if n_calls == 1 else args.workload,
              "rows": sum(c.Q for c in cases), "keys": max(c.N for c in cases), "heads": 64,
              "dim": 128, "K": cases[0].K, "pairs": pairs, "calls_per_step": n_calls,
              "launch": "graph" if args.graph else "eager"}
    roofline = {"bound": "mfma", "achieved": achieved, "peak": FP8_DENSE_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / FP8_DENSE_PEAK_TFLOPS,
                "traffic": stored_traffic("k_prefill_pair", args.workload) if n_calls == 1 else None,
                "kernel": "k_prefill_pair", "ms_per_launch": main_avg,
                "clock_ghz": clock_ghz,
                "frac_at_clock": (achieved / (FP8_DENSE_PEAK_TFLOPS * clock_ghz / NOMINAL_CLOCK_GHZ)
                                  if clock_ghz else None)}
    res = result(args, pairs / (ms_per_step * 1e-3) / 1e9, ms_per_step, config, roofline,
                 "fp8_e4m3 x fp8_e4m3 -> f32")
    res["pct_fp8_peak"] = (100.0 * pairs * FLOP_PER_PAIR / (ms_per_step * 1e-3) / 1e12
                           / FP8_DENSE_PEAK_TFLOPS)
    res["exposed_selection"] = {"control_ms_per_step": ms_control, "complete_ms_per_step": ms_per_step,
                                "control_main_ms_per_launch": control_avg,
                                "frac": (ms_per_step - ms_control) / ms_per_step}
    if n_calls > 1:
        res["subcalls"] = subcalls
    if args.workload in COLD:
        cold_ms, cold_main = timed_cold(step, args.steps)
        log("cold (512 MiB written and read back between calls): call %.4f ms, main kernel %.4f ms" % (cold_ms, cold_main))
        res["cold"] = {"ms_per_call": cold_ms, "main_ms_per_launch": cold_main,
                       "main_hbm_gbs": prefill_bytes(cases[0]) / (cold_main * 1e-3) / 1e9,
                       "warm_main_hbm_gbs": prefill_bytes(cases[0]) / (main_avg * 1e-3) / 1e9}
    if args.cpu_seconds > 0:
        res["cpu_baseline"] = cpu_baseline_prefill(cases[0], args.cpu_seconds)
    return res


def prefill_bytes(case) -> int:
    """Algorithmic HBM bytes of one prefill call: q (8 KiB), w and q_scale
    (512 B) and the output (4 B x K) per row; codes and scale of every key
    in the rows' union range once (132 B)."""
    lo, hi = int(case.row_start.min()), int(case.row_end.max())
    return int(case.Q * (64 * 128 + 2 * 64 * 4 + 4 * case.K + 8) + (hi - lo) * 132)


def bench_unfused(args, lib):
    """The unfused comparator on a prefill workload: idx_topk_prefill_unfused
    (the same scoring writes the [Q,N] FP32 matrix, then the dense top-K), the
    fused idx_topk_prefill timed the same way in the same process, and the
    standalone dense top-K (idx_topk_rows) on the matrix alone."""
    made = synth.WORKLOADS[args.workload](0)
    cases = made if isinstance(made, list) else [made]
    pairs = sum(c.pairs for c in cases)
    devs = [{k: tensor(getattr(c, k)) for k in
             ("q8", "q_scale", "k8", "k_scale", "w", "row_start", "row_end")} for c in cases]
    outs = [torch.empty((c.Q, c.K), dtype=torch.int32, device="cuda") for c in cases]
    n_calls = len(cases)
    wsu = [lib.alloc_workspace(lib.prefill_unfused_workspace_bytes(c.Q, c.N, c.K), "cuda")
           for c in cases]

    def step_unfused(step_evs, reps):
        for j, (c, d) in enumerate(zip(cases, devs)):
            lib.prefill_unfused(d["q8"], d["q_scale"], d["k8"], d["k_scale"], d["w"],
                                d["row_start"], d["row_end"], c.K, out=outs[j], workspace=wsu[j],
                                main_events=None if step_evs is None else step_evs[j], main_reps=reps)

    ms_unf, score_avg, score_min = timed(step_unfused, n_calls, args.steps, args.warmup)
    del wsu
    wsf = [lib.alloc_workspace(lib.prefill_workspace_bytes(c.Q, c.N, c.K), "cuda") for c in cases]

    def step_fused(step_evs, reps):
        for j, (c, d) in enumerate(zip(cases, devs)):
            lib.prefill_debug(d["q8"], d["q_scale"], d["k8"], d["k_scale"], d["w"], d["row_start"],
                              d["row_end"], c.K, out=outs[j], workspace=wsf[j],
                              main_events=None if step_evs is None else step_evs[j], main_reps=reps)

    ms_fused, main_avg, _ = timed(step_fused, n_calls, args.steps, args.warmup)
    # standalone dense top-K over each call's score matrix
    mats = []
    for j, (c, d) in enumerate(zip(cases, devs)):
        S = torch.empty((c.Q, c.N), dtype=torch.float32, device="cuda")
        lib.prefill_debug(d["q8"], d["q_scale"], d["k8"], d["k_scale"], d["w"], d["row_start"],
                          d["row_end"], c.K, out=outs[j], workspace=wsf[j], scores_out=S)
        mats.append(S)
    del wsf

    def step_rows(step_evs, reps):
        for j, (c, d) in enumerate(zip(cases, devs)):
            if step_evs is not None:
                step_evs[j][0].record()
            for _ in range(reps):
                lib.topk_rows(mats[j], d["row_start"], d["row_end"], c.K, out=outs[j])
            if step_evs is not None:
                step_evs[j][1].record()

    ms_rows, _, _ = timed(step_rows, n_calls, args.steps, args.warmup)
    log("workload", args.workload, "unfused ms/step %.4f (scoring %.4f)" % (ms_unf, score_avg * n_calls),
        "fused ms/step %.4f (main %.4f)" % (ms_fused, main_avg * n_calls),
        "standalone top-K ms/step %.4f" % ms_rows)
    achieved = FLOP_PER_PAIR * (pairs / n_calls) / (score_avg * 1e-3) / 1e12
    config = {"workload": cases[0].name if n_calls == 1 else args.workload, "variant": "unfused",
              "rows": sum(c.Q for c in cases), "keys": max(c.N for c in cases), "heads": 64,
              "dim": 128, "K": cases[0].K, "pairs": pairs, "calls_per_step": n_calls}
    roofline = {"bound": "mfma", "achieved": achieved, "peak": FP8_DENSE_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / FP8_DENSE_PEAK_TFLOPS, "traffic": None,
                "kernel": "k_prefill_pair (dense scores)", "ms_per_launch": score_avg}
    res = result(args, pairs / (ms_unf * 1e-3) / 1e9, ms_unf, config, roofline,
                 "fp8_e4m3 x fp8_e4m3 -> f32")
    res["compare"] = {"unfused_ms_per_step": ms_unf, "fused_ms_per_step": ms_fused,
                      "fused_speedup": ms_unf / ms_fused, "standalone_topk_ms_per_step": ms_rows,
                      "scoring_ms_per_step": score_avg * n_calls,
                      "fused_main_ms_per_step": main_avg * n_calls}
    return res


def scan_score_bytes(case) -> int:
    """Algorithmic bytes of k_scan_bf16: every scored stream (K < L <= N)
    reads its keys (256 B each), its query (64x128 BF16) and weights (64 x
    4 B), and writes one FP32 score per key; shorter streams take the remap
    path of the selection kernel and are not read."""
    n = 0
    for L in case.lens.astype(np.int64):
        if case.K < L <= case.N:
            n += L * 256 + 64 * 128 * 2 + 64 * 4 + L * 4
    return int(n)


def cpu_baseline_scan(case, seconds: float):
    """The oracle on whole streams of the workload, one after another until
    `seconds`; the rate is in key bytes per second like the GPU's."""
    import oracle
    threads = oracle_threads()
    done, dt, b = 0, 0.0, 0
    while b == 0 or dt < seconds:
        s = b % case.B
        t0 = time.perf_counter()
        oracle.scan_bf16(case.q16[s:s + 1], case.w[s:s + 1], case.k16[s:s + 1], case.lens[s:s + 1], case.K,
                         want_scores=False, nthreads=threads)
        dt += time.perf_counter() - t0
        done += int(case.lens[s])
        b += 1
    return {"value": done * 256 / dt / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "%d whole streams of %s (%d keys), fp64 exact scoring + full sort per stream, "
                      "%.1f s" % (b, case.name, done, dt)}


def bench_scan(args, lib):
    case = synth.WORKLOADS[args.workload](0)
    q16 = torch.from_numpy(case.q16.view(np.int16)).cuda()
    k16 = torch.from_numpy(case.k16.view(np.int16)).cuda()
    w = tensor(case.w)
    lens = tensor(case.lens)
    out = torch.empty((case.B, case.K), dtype=torch.int32, device="cuda")
    ws = lib.alloc_workspace(lib.scan_bf16_workspace_bytes(case.B, case.N, case.K), "cuda")

    def step(step_evs, reps):
        lib.scan_bf16(q16, w, k16, lens, case.K, out=out, workspace=ws,
                      main_events=None if step_evs is None else step_evs[0], main_reps=reps)

    ms_per_step, main_avg, main_min = timed(with_graph(args, lib, step), 1, args.steps, args.warmup)
    # the streaming floor over the same key records (one float out per key)
    floor_out = torch.empty(case.B * case.N, dtype=torch.float32, device="cuda")
    for _ in range(args.warmup):
        lib.stream_floor(k16, out=floor_out)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        lib.stream_floor(k16, out=floor_out)
    e1.record()
    torch.cuda.synchronize()
    floor_ms = e0.elapsed_time(e1) / args.steps
    key_bytes = int(case.lens.clip(0, case.N).astype(np.int64).sum()) * 256
    log("workload", args.workload, "ms/step %.4f" % ms_per_step,
        "scan kernel ms/launch %.4f (min %.4f)" % (main_avg, main_min), "floor ms %.4f" % floor_ms)
    log("  ", case.name, lib.read_stats(ws))
    nbytes = scan_score_bytes(case)
    achieved = nbytes / (main_avg * 1e-3) / 1e9
    config = {"workload": case.name, "streams": case.B, "keys_per_stream": case.N, "heads": 64, "dim": 128,
              "K": case.K, "key_bytes": key_bytes, "calls_per_step": 1,
              "launch": "graph" if args.graph else "eager"}
    roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS,
                "traffic": stored_traffic("k_scan_bf16", args.workload),
                "kernel": "k_scan_bf16", "ms_per_launch": main_avg, "algorithmic_bytes": nbytes}
    res = result(args, key_bytes / (ms_per_step * 1e-3) / 1e9, ms_per_step, config, roofline,
                 "bf16 x bf16 -> f32")
    res.update(metric=SCAN_METRIC, unit="GB/s", data="synthetic (seeded Gaussian, BF16 keys and queries)")
    res["compare"] = {"stream_floor_ms": floor_ms,
                      "stream_floor_GBs": (case.B * case.N * (256 + 4)) / (floor_ms * 1e-3) / 1e9,
                      "scan_kernel_ms": main_avg, "scan_over_floor": main_avg / floor_ms,
                      "step_over_floor": ms_per_step / floor_ms}
    if args.cpu_seconds > 0:
        res["cpu_baseline"] = cpu_baseline_scan(case, args.cpu_seconds)
    return res


def decode_score_bytes(case) -> int:
    """Algorithmic bytes of k_decode_score: every scored sequence (L > K)
    reads its keys (128 B codes + 4 B scale each), its page-table entries,
    its query (64x128 B), weights and q scales (2 x 64 x 4 B), and writes one
    FP32 score per key; shorter sequences only have their page ids checked
    (4 B per page) and take the remap path in the selection kernel."""
    n = 0
    for L in case.seq_lens.astype(np.int64):
        if L > case.K:
            n += L * 132 + ((L + 63) // 64) * 4 + 64 * 128 + 2 * 64 * 4 + L * 4
        else:
            n += ((L + 63) // 64) * 4
    return int(n)


def bench_decode(args, lib):
    case = synth.WORKLOADS[args.workload](0)
    d = {k: tensor(getattr(case, k)) for k in
         ("q8", "q_scale", "k_cache", "k_scale", "w", "page_table", "seq_lens")}
    out = torch.empty((case.B, case.K), dtype=torch.int32, device="cuda")
    ws = lib.alloc_workspace(lib.decode_workspace_bytes(case.B, case.max_pages, case.page_size,
                                                        case.K), "cuda")

    def step(step_evs, reps):
        lib.decode_paged(d["q8"], d["q_scale"], d["k_cache"], d["k_scale"], d["w"], d["page_table"],
                         d["seq_lens"], case.K, out=out, workspace=ws,
                         main_events=None if step_evs is None else step_evs[0], main_reps=reps)

    ms_per_step, main_avg, main_min = timed(with_graph(args, lib, step), 1, args.steps, args.warmup)
    log("workload", args.workload, "keys", case.pairs, "ms/step %.4f" % ms_per_step,
        "scoring kernel ms/launch %.4f (min %.4f)" % (main_avg, main_min))
    log("  ", case.name, lib.read_stats(ws))
    nbytes = decode_score_bytes(case)
    achieved = nbytes / (main_avg * 1e-3) / 1e9
    config = {"workload": case.name, "batch": case.B, "keys": case.pairs,
              "max_seq_len": int(case.seq_lens.max()), "page_size": case.page_size, "heads": 64,
              "dim": 128, "K": case.K, "pairs": case.pairs, "calls_per_step": 1,
              "launch": "graph" if args.graph else "eager"}
    roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS,
                "traffic": stored_traffic("k_decode_score", args.workload),
                "kernel": "k_decode_score", "ms_per_launch": main_avg,
                "algorithmic_bytes": nbytes}
    res = result(args, case.pairs / (ms_per_step * 1e-3) / 1e9, ms_per_step, config, roofline,
                 "fp8_e4m3 x fp8_e4m3 -> f32")
    cold_ms, cold_main = timed_cold(step, args.steps)
    log("cold (512 MiB written and read back between calls): call %.4f ms, scoring kernel %.4f ms" % (cold_ms, cold_main))
    res["cold"] = {"ms_per_call": cold_ms, "main_ms_per_launch": cold_main,
                   "main_hbm_gbs": nbytes / (cold_main * 1e-3) / 1e9,
                   "warm_main_hbm_gbs": achieved, "pairs_per_s_cold": case.pairs / (cold_ms * 1e-3)}
    if args.cpu_seconds > 0:
        res["cpu_baseline"] = cpu_baseline_decode(case, args.cpu_seconds)
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="long_prefill", choices=PREFILL + DECODE + SCAN)
    ap.add_argument("--cpu-seconds", type=float, default=30.0,
                    help="oracle sample budget in seconds (0: skip the CPU baseline)")
    ap.add_argument("--unfused", action="store_true",
                    help="time the unfused comparator (score matrix, then top-K) on a prefill "
                         "workload, beside the fused path and the standalone top-K")
    ap.add_argument("--graph", action="store_true",
                    help="replay each step's library calls from a HIP graph recorded once "
                         "(idx_topk_graph_*) instead of launching them one by one")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain copy of MIB MiB (counter calibration) and exit")
    args = ap.parse_args()
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    import scoring_exact_top_amd as lib
    if args.unfused:
        if args.workload not in PREFILL:
            print("--unfused applies to prefill workloads", file=sys.stderr)
            sys.exit(2)
        res = bench_unfused(args, lib)
    else:
        res = (bench_decode if args.workload in DECODE else
               bench_scan if args.workload in SCAN else bench_prefill)(args, lib)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of the skinny decode linear on one MI355X.

Workload: the bf16 decode-linear sweep -- M in {1,2,3,4,6,8,12,16,24,32,64,96,
128} x (N, K) in {(4096,4096), (6144,4096), (4096,12288), (2048,2048),
(1024,1024)}, x ~ N(0,1), W ~ N(0,0.02), seed 0.  One step is one pass of the
whole path over that sweep: 65 calls of skinny_gemm_bf16_packed through the
library's table dispatch, each weight packed once (skinny_gemm_pack_weight)
before timing, as a deployment packs it at load.  The same step on row-major
weights (skinny_gemm_bf16) is timed in the same run and reported beside the
value.  Inputs are resident in HBM before timing starts.  Each shape
cycles through enough copies of W (>= 1 GiB per shape) that every call streams
its weight from HBM, not from the 256 MB Infinity Cache.  Steps are replayed
from HIP graphs, eight steps per graph.  The dominant kernel's launches of
those steps are grouped in their own graph and bracketed by HIP events on the
launch stream, which gives its live average duration for the roofline figure.
Beside the nominal peaks it reports what a kernel can reach on the device: the
fastest plain read of each shape's rotated weight copies and the rate of a
register-only bf16 MFMA loop (the library's measurement kernels).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--detail PATH] [--verbose]

Prints one compact JSON line on stdout (the headline metric, the dominant
kernel's roofline, the CPU oracle's rate and the M = 1/8/128 calls); the
per-call, mid-M, small-N and other-form reports go to the file named by
--detail.  Progress goes to stderr with --verbose.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA
READ_GRIDS = (512, 1024, 2048, 4096, 8192)   # workgroup counts tried for a read ceiling
METRIC = "achieved HBM GB/s and µs/call at M=1/8/128; fraction of MI355X roofline"


VERBOSE = False


def log(*a):
    if VERBOSE:
        print(*a, file=sys.stderr, flush=True)


def alg_bytes(M, N, K):
    """Algorithmic bytes of one bf16 call: W once, x once, y once."""
    return 2 * N * K + 2 * M * K + 2 * M * N


def kernel_symbol(variant: str, M: int, op: int = 0) -> str:
    """The kernel template instance a variant runs for M rows, as rocprofv3
    prints it.  Variant names are the family followed by one-letter fields:
    gemv_r<R>_k<KS>_p<P>, tile_f<FN>_k<KS>_p<P>, and
    tlds[_d|_x][_w<NW>][_k<KW>]_f<FN>_s<S>_p<P>[_m<MC>] (d: direct x; x: x copied
    into LDS by DMA; NW waves,
    default 4, of which KW split K inside the workgroup, default 1; at most MC
    16-row fragments per workgroup, default 8), and the two-operand tile
    mt_m<FM>_f<FN>_a<WM>_b<WN>_s<S>_p<P>, and the packed-weight stream
    pg_r<RW>_k<KS>_p<P>."""
    parts = variant.split("_")
    if parts[0] == "pg":                      # pg_r<RW>_k<KS>_p<P>
        kv = {p[0]: int(p[1:]) for p in parts[1:]}
        mt = next(b for b in (1, 2, 3, 4, 6, 8, 12, 16) if M <= b)
        return f"void skg::pg_kernel<{op}, {mt}, {kv['r']}, {kv['k']}, {kv['p']}>(skg::Args)"
    if parts[0] == "mt":                      # mt_m<FM>_f<FN>_a<WM>_b<WN>_s<S>_p<P>
        kv = {p[0]: int(p[1:]) for p in parts[1:]}
        return (f"void skg::mt_kernel<{op}, {kv['m']}, {kv['f']}, {kv['a']}, {kv['b']}, {kv['s']}, "
                f"{kv['p']}>(skg::Args)")
    xd = 1 if "d" in parts[1:] else (2 if "x" in parts[1:] else 0)
    kv = {p[0]: int(p[1:]) for p in parts[1:] if p not in ("d", "x")}
    if parts[0] == "gemv":
        mt = next(b for b in (1, 2, 3, 4, 6, 8, 12, 16) if M <= b)
        return f"void skg::gemv_kernel<{op}, {mt}, {kv['r']}, {kv['k']}, {kv['p']}>(skg::Args)"
    f = (min(M, 128) + 15) // 16
    fm = next(b for b in (1, 2, 4, 6, 8) if f <= b)
    if parts[0] == "tile":
        return f"void skg::tile_kernel<{op}, {fm}, {kv['f']}, {kv['k']}, {kv['p']}>(skg::Args)"
    fm = min(fm, kv.get("m", 8))
    return (f"void skg::tlds_kernel<{op}, {fm}, {kv['f']}, {kv['s']}, {kv['p']}, {kv.get('w', 4)}, "
            f"{kv.get('k', 1)}, {xd}>(skg::Args)")


def lib_code_hash() -> str:
    """Hash of the kernel and dispatch sources the library was built from."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gemv_skinny_gemm_02_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def read_counters(kernel: str, code_hash: str):
    """HBM traffic per launch of `kernel` from the committed counter summary,
    if it was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "bf16_sweep_counters.txt")
    if not os.path.exists(path):
        return None
    kv, rows = {}, {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("kernel "):
                _, rest = line.split(" ", 1)
                name, fetch, write = rest.rsplit("|", 2)
                rows[name.strip()] = (float(fetch), float(write))
            elif "=" in line:
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("code_hash") != code_hash or kernel not in rows:
        return None
    ff, wf = float(kv["copy_fetch_factor"]), float(kv["copy_write_factor"])
    fetch_kib, write_kib = rows[kernel]
    return (fetch_kib / ff + write_kib / wf) * 1024.0


def host_cores() -> int:
    """CPU cores this process may run on."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def blas_threads() -> int:
    """Threads of the BLAS pool the oracle's float64 products run on."""
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        return int(os.environ.get("OMP_NUM_THREADS", "1"))


def cpu_baseline(calls, host, seconds: float, runs: int = 3):
    """The oracle, as it stands, run over the step's calls in step order, pass
    after pass, for `seconds` of wall time per run (the last pass may stop
    part-way): the median of `runs` runs, in algorithmic bytes per second.
    Beside it, the two parts of the oracle's work timed apart on one weight of
    each shape: decoding the bf16 weight to float64, and the float64 product
    (one call at M = 8)."""
    import oracle
    rates, ncalls_all = [], []
    for _ in range(runs):
        ncalls, nbytes, t0 = 0, 0, time.perf_counter()
        done = False
        while not done:
            for (M, N, K) in calls:
                xb, wb = host[(N, K)]
                oracle.linear_bf16(xb[:M], wb)
                nbytes += alg_bytes(M, N, K)
                ncalls += 1
                if time.perf_counter() - t0 >= seconds:
                    done = True
                    break
        rates.append(nbytes / (time.perf_counter() - t0) / 1e9)
        ncalls_all.append(ncalls)
    split = {}
    for (N, K), (xb, wb) in host.items():
        t0 = time.perf_counter()
        wd = oracle.dec_bf16(wb)
        t1 = time.perf_counter()
        _ = oracle.dec_bf16(xb[:8]) @ wd.T
        t2 = time.perf_counter()
        split[f"{N}x{K}"] = {"decode_s": round(t1 - t0, 4), "product_s_M8": round(t2 - t1, 4)}
        del wd
    threads = min(blas_threads(), host_cores())
    return {"value": round(statistics.median(rates), 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"median of {runs} runs of {seconds:.0f} s, each the step's {len(calls)} calls in order "
                      f"({min(ncalls_all)}-{max(ncalls_all)} calls), oracle.linear_bf16 in float64 on "
                      f"{threads} BLAS threads of {host_cores()} host cores",
            "runs_GBs": [round(r, 4) for r in rates], "decode_vs_product": split}


def cpu_oracle_per_config(seconds: float):
    """The oracle, as it stands, on one call of each form at M = 1, each on a
    row sample of its weight (the oracle's work is per weight row), repeated
    for `seconds` with one BLAS thread and with all of them; algorithmic bytes
    of the sampled call per second."""
    import oracle
    import synth
    from threadpoolctl import threadpool_limits
    all_threads = min(blas_threads(), host_cores())
    cases = [
        ("bf16 4096x4096", "bf16", synth.make_bf16(1, 4096, 4096, seed=0), 4096,
         lambda p: oracle.linear_bf16(p.x, p.w)),
        ("gated 12288x4096 (2048 of 12288 rows)", "gated", synth.make_gated(1, 2048, 4096, seed=0), 2048,
         lambda p: oracle.linear_gated(p.x, p.w)),
        ("fp8 head 248320x4096 (8192 of 248320 rows)", "fp8_tensor", synth.make_fp8_tensor(1, 8192, 4096, seed=0), 8192,
         lambda p: oracle.linear_fp8_tensor(p.x, p.w, p.s0)),
        ("a8w8 8192x4096", "a8w8_block", synth.make_a8w8_block(1, 8192, 4096, seed=0), 8192,
         lambda p: oracle.linear_a8w8_block(p.x, p.s0, p.w, p.s1)),
        ("a8w8, x quantised, 8192x4096", "a8w8_quant", synth.make_a8w8_quant(1, 8192, 4096, seed=0), 8192,
         lambda p: oracle.linear_a8w8_quant(p.x, p.w, p.s1)),
    ]
    out = {}
    for name, form, p, n_rows, fn in cases:
        nbytes = alg_bytes(1, n_rows, 4096) if form == "bf16" else form_alg_bytes(form, 1, n_rows, 4096)
        row = {"sample": f"M=1, {n_rows} weight rows, K=4096", "alg_bytes": nbytes}
        for threads in (1, all_threads):
            with threadpool_limits(limits=threads, user_api="blas"):
                calls, t0 = 0, time.perf_counter()
                while calls == 0 or time.perf_counter() - t0 < seconds:
                    fn(p)
                    calls += 1
                dt = time.perf_counter() - t0
            row[f"GB/s_{threads}_threads"] = round(nbytes * calls / dt / 1e9, 4)
        out[name] = row
    return {"threads": all_threads, "configs": out}


WORKLOAD = ("bf16 decode-linear sweep, seed 0: M in {1,2,3,4,6,8,12,16,24,32,64,96,128} x (N,K) in "
            "{4096x4096, 6144x4096, 4096x12288, 2048x2048, 1024x1024}, x~N(0,1), W~N(0,0.02), 65 calls/step, "
            "packed weights rotated past the Infinity Cache")


def make_line(value, ms_step, steps, warmup, ncalls, roofline, per_m, cpu=None) -> dict:
    """The one JSON line the benchmark prints: the headline metric and its
    configuration, the dominant kernel's roofline, the M = 1/8/128 calls as
    [µs, GB/s] per shape, and the CPU oracle's rate (added when measured).
    Everything else goes to the detail file, so that the line stays short."""
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "calls_per_step": ncalls},
        "roofline": roofline,
        "per_m_us_gbs": per_m,
    }
    if cpu is not None:
        line["cpu_baseline"] = cpu
    return line


def measure_step(args, torch, skg, calls, Ms, stream, launch, op, step_bytes):
    """Time args.steps steps of `calls` launched by `launch(call, copy)` (table
    dispatch of form `op`): returns the step time, its rate and the dominant
    kernel's live average launch time."""
    choice = {c: skg.skinny_gemm_query(op, *c) for c in calls}
    sym = {c: kernel_symbol(choice[c][0], c[0], skg.OPS[op]) for c in calls}
    for c in calls:                      # eager warm-up (and lazy table load)
        launch(c, 0)
    torch.cuda.synchronize()

    # ------------------- which kernel dominates a step (3 eager timings each)
    rough_us = {}
    for c in calls:
        ts = []
        for i in range(3):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            launch(c, 1 + i)
            b.record(stream)
            b.synchronize()
            ts.append(a.elapsed_time(b) * 1e3)
        rough_us[c] = min(ts)
    sym_time = {}
    for c in calls:
        sym_time[sym[c]] = sym_time.get(sym[c], 0.0) + rough_us[c]
    dominant = max(sym_time, key=sym_time.get)
    dom_calls = [c for c in calls if sym[c] == dominant]
    rest_calls = [c for c in calls if sym[c] != dominant]
    log(f"dominant kernel {dominant}: {len(dom_calls)} calls/step, ~{sym_time[dominant]:.1f} us/step")

    # ---------------------------------------------------------- step graphs
    # Steps are replayed in blocks of B: one graph holds the non-dominant calls
    # of B steps, another the dominant kernel's calls of the same B steps, so
    # each HIP event pair brackets B * len(dom_calls) back-to-back launches and
    # the graph-launch boundary is amortised.  Step s of a block uses weight
    # copy (s * len(Ms) + i) for the i-th M of a shape.
    B = max(1, min(8, args.steps))
    nM = len(Ms)

    def capture(subset, steps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for s_ in steps:
                for c in subset:
                    launch(c, s_ * nM + Ms.index(c[0]))
        return g

    g_rest = capture(rest_calls, range(B))
    g_dom = capture(dom_calls, range(B))
    rem = args.steps % B
    g_rest_r = capture(rest_calls, range(rem)) if rem else None
    g_dom_r = capture(dom_calls, range(rem)) if rem else None
    torch.cuda.synchronize()

    for _ in range(max(1, args.warmup // B)):
        g_rest.replay()
        g_dom.replay()
    torch.cuda.synchronize()

    # ------------------------------------------------------- timed steps
    blocks = args.steps // B
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(blocks + (1 if rem else 0))]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for bi in range(blocks):
        g_rest.replay()
        pairs[bi][0].record(stream)
        g_dom.replay()
        pairs[bi][1].record(stream)
    if rem:
        g_rest_r.replay()
        pairs[-1][0].record(stream)
        g_dom_r.replay()
        pairs[-1][1].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t_start.elapsed_time(t_end) / args.steps
    dom_us = sum(e0.elapsed_time(e1) for e0, e1 in pairs) * 1e3 / (args.steps * len(dom_calls))
    value = step_bytes / (ms_step * 1e-3) / 1e9
    log(f"{op}: step {ms_step * 1e3:.1f} us ({wall / args.steps * 1e6:.1f} us wall), {value:.1f} GB/s, "
        f"dominant kernel {dom_us:.2f} us/launch")

    del g_rest, g_dom, g_rest_r, g_dom_r
    return {"launch": launch, "choice": choice, "dominant": dominant, "dom_calls": dom_calls,
            "rough_us": rough_us, "ms_step": ms_step, "dom_us": dom_us, "value": value}


_WS_BYTES = [0]


def ensure_ws(skg, need: int) -> None:
    """Register a larger device split-K workspace when `need` exceeds the
    current one (the binding keeps the old one alive)."""
    if need > _WS_BYTES[0]:
        skg.skinny_gemm_set_device_workspace(max(need, 1 << 20))
        _WS_BYTES[0] = max(need, 1 << 20)


def _graph_us(torch, stream, n, enqueue, replays):
    """Median µs per launch of a graph of n launches enqueue(i)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            enqueue(i)
    g.replay()
    torch.cuda.synchronize()
    ts = []
    for _ in range(max(1, replays)):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        g.replay()
        b.record(stream)
        b.synchronize()
        ts.append(a.elapsed_time(b) * 1e3 / n)
    del g
    return statistics.median(ts)


def measure_ceilings(args, torch, skg, shapes, wp_dev, stream):
    """What a kernel can reach here: per weight size, the fastest plain read of
    the same rotated weight copies (the library's read-stream kernel, graph
    replay as for the calls, best of five grid sizes); and the bf16 MFMA rate
    of a register-only MFMA loop on every CU."""
    sink = torch.empty(256, dtype=torch.int32, device="cuda")
    read = {}
    for (N, K) in shapes:
        bufs = [w.data for w in wp_dev[(N, K)]]
        R = len(bufs)
        n = max(args.per_call_min, 2 * R)
        best = None
        for grid in READ_GRIDS:
            for sweep in (False, True):
                us = _graph_us(torch, stream, n,
                               lambda i: skg.skinny_gemm_calib_read(bufs[i % R], grid, sink, sweep=sweep),
                               args.per_call_replays)
                if best is None or us < best[0]:
                    best = (us, grid, sweep)
        nbytes = bufs[0].numel()
        read[(N, K)] = {"bytes": nbytes, "us": round(best[0], 3), "GB/s": round(nbytes / (best[0] * 1e-6) / 1e9, 1),
                        "grid": best[1], "order": "sweep" if best[2] else "slices"}
    grid, iters = 8 * 256, 2048
    flops = skg.skinny_gemm_calib_mfma(grid, iters, sink)       # warm-up
    torch.cuda.synchronize()
    ts = []
    for _ in range(3):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        skg.skinny_gemm_calib_mfma(grid, iters, sink)
        b.record(stream)
        b.synchronize()
        ts.append(a.elapsed_time(b) * 1e-3)
    mfma_tflops = flops / min(ts) / 1e12
    log("read ceilings:", {f"{N}x{K}": v["us"] for (N, K), v in read.items()}, f"| mfma bf16 {mfma_tflops:.0f} TFLOP/s")
    return {"read": read, "mfma_bf16_tflops": mfma_tflops}


def measure_host_cost(torch, skg, x_dev, wp_dev, y_dev, stream, n=2000):
    """Host cost of an eager call: µs per launch of n back-to-back launches
    from the host (no graph), for a near-empty kernel (one workgroup of the
    MFMA measurement kernel) and for the packed bf16 call on 1024 x 1024 at
    M = 1, each through the Python binding and through the bare C entry
    point with its arguments prepared once."""
    lib = skg.load()
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    M, N, K = 1, 1024, 1024
    x, wp, y = x_dev[K][:M], wp_dev[(N, K)][0], y_dev[(M, N)]
    sp = stream.cuda_stream
    xp, wpp, yp, skp = x.data_ptr(), wp.data.data_ptr(), y.data_ptr(), sink.data_ptr()

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        host_us = (time.perf_counter() - t0) * 1e6 / n
        b.synchronize()
        return round(a.elapsed_time(b) * 1e3 / n, 3), round(host_us, 3)

    rows = {
        "empty_kernel_binding": timed(lambda: skg.skinny_gemm_calib_mfma(1, 1, sink)),
        "empty_kernel_c": timed(lambda: lib.skinny_gemm_calib_mfma(1, 1, skp, sp)),
        "bf16_packed_1024_M1_binding": timed(lambda: skg.skinny_gemm_bf16_packed(x, wp, y=y)),
        "bf16_packed_1024_M1_c": timed(lambda: lib.skinny_gemm_bf16_packed(xp, wpp, None, yp, M, N, K, sp)),
    }
    return {"launches": n, "unit": "µs per launch: (device events, host issue time)", "rows": rows}


def measure_mid_m(args, torch, skg, synth, shapes, wp_dev, stream, ceil):
    """Mid-M rows (speculative verification and drafting) on the sweep shapes:
    µs per call of the packed form through table dispatch, graph replay over
    the same rotated weight copies as the step.  As context, the vendor GEMM
    (torch.mm of x and the transposed weight, hipBLASLt) timed the same way on
    the same buffers read as row-major [N, K] bf16 weights: its speed does not
    depend on the values, so no further copies are needed."""
    out = {}
    Mmax = max(synth.MID_M)
    ensure_ws(skg, max(skg.skinny_gemm_workspace_bytes("bf16_packed", M, N, K) for (N, K) in shapes for M in synth.MID_M))
    for (N, K) in shapes:
        x = torch.from_numpy(synth.make_bf16(Mmax, 16, K, seed=0).x.view(np.int16)).view(torch.bfloat16).cuda()
        ws = wp_dev[(N, K)]
        R = len(ws)
        n = max(args.per_call_min, 2 * R)
        rm = [w.data.view(torch.bfloat16).view(N, K) for w in ws]
        row = {}
        for M in synth.MID_M:
            xm = x[:M]
            y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
            ours = _graph_us(torch, stream, n, lambda i: skg.skinny_gemm_bf16_packed(xm, ws[i % R], y=y),
                             args.per_call_replays)
            torch.mm(xm, rm[0].t(), out=y)           # the vendor library sets itself up outside capture
            torch.cuda.synchronize()
            vendor = _graph_us(torch, stream, n, lambda i: torch.mm(xm, rm[i % R].t(), out=y), args.per_call_replays)
            nbytes = alg_bytes(M, N, K)
            tfl = 2 * M * N * K / (ours * 1e-6) / 1e12
            floor_us = max(ceil["read"][(N, K)]["us"], 2 * M * N * K / (ceil["mfma_bf16_tflops"] * 1e12) * 1e6)
            row[str(M)] = {"us": round(ours, 2), "GB/s": round(nbytes / (ours * 1e-6) / 1e9, 1),
                           "TFLOP/s": round(tfl, 1), "hbm_frac": round(nbytes / (ours * 1e-6) / 1e9 / HBM_PEAK_GBS, 3),
                           "mfma_frac": round(tfl / MFMA_BF16_PEAK_TFLOPS, 4),
                           "ceiling_frac": round(floor_us / ours, 3),
                           "variant": skg.skinny_gemm_query("bf16_packed", M, N, K)[0],
                           "vendor_us": round(vendor, 2)}
        out[f"{N}x{K}"] = row
        log(f"mid-M {N}x{K}:", {m: (v["us"], v["vendor_us"]) for m, v in row.items()})
    return {"rows": list(synth.MID_M), "form": "bf16_packed, table dispatch", "shapes": out,
            "ceiling": "max(read time of the weight, flops at the MFMA-loop rate)",
            "vendor": "torch.mm (hipBLASLt), bf16, same rotated buffers, graph replay: context only"}


def measure_small_n(args, torch, skg, synth, stream):
    """Small-N bf16 weights (N = 64 .. 2048, K = 4096): µs per call of both
    layouts through table dispatch, and the read ceiling of each weight, all
    in graph replay over >= 1 GiB of rotated copies."""
    sink = torch.empty(256, dtype=torch.int32, device="cuda")
    out = {}
    Mmax = max(synth.SMALLN_M)
    ensure_ws(skg, max(skg.skinny_gemm_workspace_bytes(op, M, N, K) for (N, K) in synth.SMALLN_NK
                       for M in synth.SMALLN_M for op in ("bf16", "bf16_packed")))
    for (N, K) in synth.SMALLN_NK:
        p = synth.make_bf16(Mmax, N, K, seed=0)
        x = torch.from_numpy(p.x.view(np.int16)).view(torch.bfloat16).cuda()
        w0 = torch.from_numpy(p.w.view(np.int16)).view(torch.bfloat16).cuda()
        R = max(2, math.ceil(args.rotation_gib * 2**30 / (2 * N * K)))
        ws = [w0] + [w0.clone() for _ in range(R - 1)]
        wps = [skg.skinny_gemm_pack_weight("bf16", w0) for _ in range(R)]
        n = max(args.per_call_min, 2 * R)
        ceil_us = min(_graph_us(torch, stream, n, lambda i: skg.skinny_gemm_calib_read(ws[i % R], g, sink, sweep=sw),
                                args.per_call_replays) for g in (256, 512, 1024) for sw in (False, True))
        row = {}
        for M in synth.SMALLN_M:
            xm = x[:M]
            y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
            rm = _graph_us(torch, stream, n, lambda i: skg.skinny_gemm_bf16(xm, ws[i % R], y=y), args.per_call_replays)
            pk = _graph_us(torch, stream, n, lambda i: skg.skinny_gemm_bf16_packed(xm, wps[i % R], y=y),
                           args.per_call_replays)
            row[str(M)] = {"row_major_us": round(rm, 2), "packed_us": round(pk, 2),
                           "read_ceiling_frac": round(ceil_us / min(rm, pk), 3),
                           "row_major_variant": skg.skinny_gemm_query("bf16", M, N, K)[0],
                           "packed_variant": skg.skinny_gemm_query("bf16_packed", M, N, K)[0]}
        out[f"{N}x{K}"] = {"read_ceiling_us": round(ceil_us, 3), "rows": row}
        log(f"small-N {N}x{K}: ceiling {ceil_us:.2f} us,", {m: (v["row_major_us"], v["packed_us"]) for m, v in row.items()})
        del ws, wps, w0
        torch.cuda.empty_cache()
    return {"form": "bf16, table dispatch, row-major and packed", "shapes": out,
            "read_ceiling_frac": "read ceiling of the weight / the faster layout's call"}


def form_alg_bytes(form, M, N, K):
    """Algorithmic bytes of one call of a form: the weight once (gate and up
    rows for the gated form), x once, its scales once, y once."""
    kb, nb = -(-K // 128), -(-N // 128)
    if form == "gated":
        return 4 * N * K + 2 * M * K + 2 * M * N
    if form == "fp8_tensor":
        return N * K + 2 * M * K + 2 * M * N + 4
    if form == "a8w8_quant":          # bf16 x in; the x scales are not handed out here
        return N * K + 2 * M * K + 4 * nb * kb + 2 * M * N
    return N * K + M * K + 4 * M * kb + 4 * nb * kb + 2 * M * N


def form_operands(torch, gen, form, N, K, Mmax):
    """Device operands (x [Mmax, K], the row-major weight, s0, s1) of one form
    at one shape, drawn on the device from torch's seeded generator `gen` with
    the workload distributions (x ~ N(0,1), W ~ N(0,0.02), fp8 scales
    amax/448): the values do not change the time of these kernels, and the
    oracle checks them in the tests."""
    def normal(shape, std):
        return torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32) * std

    def e4m3(v, rows, cols):
        # per-block scale amax/448 over [rows, cols] blocks of v, and the codes
        R_, C_ = v.shape
        pr, pc = -(-R_ // rows) * rows, -(-C_ // cols) * cols
        vp = torch.zeros((pr, pc), device="cuda")
        vp[:R_, :C_] = v
        blk = vp.view(pr // rows, rows, pc // cols, cols)
        sc = blk.abs().amax(dim=(1, 3)) / 448.0
        sc = torch.where(sc > 0, sc, torch.ones_like(sc))
        q = (blk / sc[:, None, :, None]).clamp(-448, 448).view(pr, pc)[:R_, :C_]
        return q.to(torch.float8_e4m3fn).contiguous(), sc.float().contiguous()

    s0 = s1 = None
    if form == "bf16":
        w0 = normal((N, K), 0.02).to(torch.bfloat16)
    elif form == "gated":
        w0 = normal((2 * N, K), 0.02).to(torch.bfloat16)
    elif form == "fp8_tensor":
        # drawn twice in the same row blocks from the same seed (the fp32
        # weight would be 4 GB): once for amax, once to quantise
        w0 = torch.empty((N, K), dtype=torch.float8_e4m3fn, device="cuda")
        amax = torch.zeros((), device="cuda")
        gen.manual_seed(1)
        for r0 in range(0, N, 16384):
            amax = torch.maximum(amax, normal((min(16384, N - r0), K), 0.02).abs().max())
        sc = (amax / 448.0).reshape(1).float()
        gen.manual_seed(1)
        for r0 in range(0, N, 16384):
            w0[r0:r0 + 16384] = (normal((min(16384, N - r0), K), 0.02) / sc).clamp(-448, 448).to(torch.float8_e4m3fn)
        s0 = sc
    else:
        w0, s1 = e4m3(normal((N, K), 0.02), 128, 128)
    xf = normal((Mmax, K), 1.0)
    if form == "a8w8_block":
        x, s0 = e4m3(xf, 1, 128)
    else:
        x = xf.to(torch.bfloat16)
    return x, w0, s0, s1


def form_call(skg, form, packed, xm, w, s0m, s1, y):
    """One call of a form's entry point (row-major or packed weight)."""
    sfx = "_packed" if packed else ""
    if form == "bf16":
        return getattr(skg, "skinny_gemm_bf16" + sfx)(xm, w, y=y)
    if form == "gated":
        return getattr(skg, "skinny_gemm_gated" + sfx)(xm, w, y=y)
    if form == "fp8_tensor":
        return getattr(skg, "skinny_gemm_fp8_tensor" + sfx)(xm, w, s0m, y=y)
    if form == "a8w8_block":
        return getattr(skg, "skinny_gemm_a8w8_block" + sfx)(xm, w, s0m, s1, y=y)
    return getattr(skg, "skinny_gemm_a8w8_block_quant" + sfx)(xm, w, s1, y=y)


def measure_forms(args, torch, skg, synth, stream):
    """The other forms at their workload shapes: gate/up 12288 x 4096, the
    248320 x 4096 fp8 head, and A8W8 (and A8W8 with x quantised in the call) at
    (32768, 1024) and (8192, 4096), A8W8 also at the mid-M rows 144 .. 512.  µs per call of the row-major and packed
    weights through table dispatch, graph replay over >= 1 GiB of rotated
    weight copies, against the read ceiling of the weight (operands from
    form_operands)."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    sink = torch.empty(256, dtype=torch.int32, device="cuda")
    cases = [("gated", synth.GATED_NK, synth.GATED_M), ("fp8_tensor", synth.HEAD_NK, synth.HEAD_M)]
    cases += [("a8w8_block", nk, tuple(synth.A8W8_M) + tuple(synth.MID_M)) for nk in synth.A8W8_NK]
    cases += [("a8w8_quant", nk, synth.A8W8_M) for nk in synth.A8W8_NK]
    out = {}
    for form, (N, K), Ms in cases:
        Mmax = max(Ms)
        ensure_ws(skg, max(skg.skinny_gemm_workspace_bytes(op, M, N, K) for M in Ms
                           for op in (form, form + "_packed")))
        x, w0, s0, s1 = form_operands(torch, gen, form, N, K, Mmax)
        wbytes = w0.numel() * w0.element_size()
        R = max(2, math.ceil(args.rotation_gib * 2**30 / wbytes))
        ws = [w0] + [w0.clone() for _ in range(R - 1)]
        wps = [skg.skinny_gemm_pack_weight(form, w0) for _ in range(R)]
        n = max(args.per_call_min, 2 * R)
        ceil_us = min(_graph_us(torch, stream, n, lambda i: skg.skinny_gemm_calib_read(ws[i % R], g, sink, sweep=sw),
                                args.per_call_replays) for g in READ_GRIDS for sw in (False, True))
        rows = {}
        for M in Ms:
            xm = x[:M]
            s0m = s0[:M] if form == "a8w8_block" else s0
            y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
            f_rm = lambda i: form_call(skg, form, False, xm, ws[i % R], s0m, s1, y)
            f_pk = lambda i: form_call(skg, form, True, xm, wps[i % R], s0m, s1, y)
            rm = _graph_us(torch, stream, n, f_rm, args.per_call_replays)
            pk = _graph_us(torch, stream, n, f_pk, args.per_call_replays)
            best = min(rm, pk)
            gbs = form_alg_bytes(form, M, N, K) / (best * 1e-6) / 1e9
            rows[str(M)] = {"row_major_us": round(rm, 2), "packed_us": round(pk, 2), "GB/s": round(gbs, 1),
                            "hbm_frac": round(gbs / HBM_PEAK_GBS, 3), "read_ceiling_frac": round(ceil_us / best, 3)}
        key = f"{form} {N}x{K}"
        out[key] = {"weight_bytes": wbytes, "read_ceiling_us": round(ceil_us, 3), "rows": rows}
        log(f"{key}: ceiling {ceil_us:.2f} us,", {m: (v["row_major_us"], v["packed_us"]) for m, v in rows.items()})
        del ws, wps, w0, x
        torch.cuda.empty_cache()
    return {"dispatch": "table", "GB/s": "algorithmic bytes / the faster layout's µs", "shapes": out}


PROFILE_FORMS = ("bf16", "gated", "fp8_tensor", "a8w8_block", "a8w8_quant", "mid_m", "small_n")


def profile_form(args, torch, skg, synth) -> int:
    """A run for the profiler: the workload calls of one form on packed weights
    through table dispatch, launched eagerly one after another (no graphs), so
    that every dispatch a profiler records is one call of the list written to
    --calls-out in launch order (with its algorithmic bytes; the first launch of
    each call is marked as a warm-up).  Each shape cycles through >= 1 GiB of
    packed weight copies.  Ends with the 256 MiB device copy the counter
    summaries calibrate on."""
    import json as _json
    form = args.profile_form
    if form == "mid_m":
        groups = [("bf16", nk, synth.MID_M) for nk in synth.SWEEP_NK]
        groups += [("a8w8_block", nk, synth.MID_M) for nk in synth.A8W8_NK]
    elif form == "small_n":
        groups = [("bf16", nk, synth.SMALLN_M) for nk in synth.SMALLN_NK]
    elif form == "bf16":
        groups = [("bf16", nk, synth.SWEEP_M) for nk in synth.SWEEP_NK]
    elif form == "gated":
        groups = [("gated", synth.GATED_NK, synth.GATED_M)]
    elif form == "fp8_tensor":
        groups = [("fp8_tensor", synth.HEAD_NK, synth.HEAD_M)]
    else:
        groups = [(form, nk, synth.A8W8_M) for nk in synth.A8W8_NK]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    launches = []
    for f, (N, K), Ms in groups:
        ensure_ws(skg, max(skg.skinny_gemm_workspace_bytes(f + "_packed", M, N, K) for M in Ms))
        x, w0, s0, s1 = form_operands(torch, gen, f, N, K, max(Ms))
        wbytes = w0.numel() * w0.element_size()
        R = max(2, math.ceil(args.rotation_gib * 2**30 / wbytes))
        wps = [skg.skinny_gemm_pack_weight(f, w0) for _ in range(R)]
        del w0
        ys = {M: torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for M in Ms}
        torch.cuda.synchronize()
        i = 0
        for p in range(args.steps + 1):
            for M in Ms:
                form_call(skg, f, True, x[:M], wps[i % R], s0[:M] if f == "a8w8_block" else s0, s1, ys[M])
                i += 1
                nb = alg_bytes(M, N, K) if f == "bf16" else form_alg_bytes(f, M, N, K)
                launches.append({"op": f + "_packed", "M": M, "N": N, "K": K, "alg_bytes": nb, "warm": p == 0,
                                 "variant": skg.skinny_gemm_query(f + "_packed", M, N, K)[0]})
        torch.cuda.synchronize()
        del wps, x, ys
        torch.cuda.empty_cache()
    src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    if args.calls_out:
        os.makedirs(os.path.dirname(os.path.abspath(args.calls_out)), exist_ok=True)
        with open(args.calls_out, "w") as fh:
            _json.dump({"form": form, "launches": launches}, fh)
    print(_json.dumps({"profile_form": form, "launches": len(launches), "passes": args.steps + 1}), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--rotation-gib", type=float, default=1.0, help="bytes of W copies per shape")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--per-call-replays", type=int, default=7, help="graph replays per call shape")
    ap.add_argument("--no-per-call", action="store_true",
                    help="skip the per-call graph timings (profiling runs: keeps every dispatch of a kernel "
                         "in the step's shape mix)")
    ap.add_argument("--per-call-min", type=int, default=64, help="min launches per per-call graph")
    ap.add_argument("--no-mid-m", action="store_true", help="skip the mid-M rows (144..512) report")
    ap.add_argument("--no-small-n", action="store_true", help="skip the small-N (N = 64..2048) report")
    ap.add_argument("--no-forms", action="store_true", help="skip the gated / fp8 head / A8W8 report")
    ap.add_argument("--no-row-major", action="store_true",
                    help="skip the row-major step (profiling runs of the packed layout)")
    ap.add_argument("--detail", default=None, help="write the full report (JSON) to this file")
    ap.add_argument("--profile-form", choices=PROFILE_FORMS, default=None,
                    help="profiler run: one form's workload calls, eager, in a recorded order (see --calls-out)")
    ap.add_argument("--calls-out", default=None, help="with --profile-form: where to write the launch list")
    ap.add_argument("--verbose", action="store_true", help="progress on stderr")
    args = ap.parse_args()
    global VERBOSE
    VERBOSE = args.verbose
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: the skinny linear is measured on one MI355X "
              "(a multi-GPU run would shard N with no exchange; see the design notes)", file=sys.stderr)
        return 2

    import torch

    import gemv_skinny_gemm_02_amd as skg
    import synth

    if not torch.cuda.is_available():
        log("no GPU")
        return 1
    torch.cuda.set_device(0)
    skg.load()
    if args.profile_form:
        return profile_form(args, torch, skg, synth)
    props = torch.cuda.get_device_properties(0)
    dev_name = f"{props.gcnArchName.split(':')[0]} ({props.multi_processor_count} CUs)"
    log("device", dev_name, "| identity", skg.skinny_gemm_identity())

    shapes = list(synth.SWEEP_NK)
    Ms = list(synth.SWEEP_M)
    calls = [(M, N, K) for (N, K) in shapes for M in Ms]

    # ---------------------------------------------------------- inputs
    host, x_dev, w_dev, wp_dev, y_dev = {}, {}, {}, {}, {}
    free, _ = torch.cuda.mem_get_info()
    need = sum(max(2, math.ceil(args.rotation_gib * 2**30 / (2 * N * K))) * 2 * N * K for N, K in shapes)
    need *= 1 if args.no_row_major else 2
    if need > 0.8 * free:
        log(f"not enough device memory for the rotation copies ({need / 2**30:.1f} GiB needed)")
        return 1
    for (N, K) in shapes:
        p = synth.make_bf16(max(Ms), N, K, seed=0)
        host[(N, K)] = (p.x, p.w)
        if K not in x_dev:
            x_dev[K] = torch.from_numpy(p.x.view(np.int16)).view(torch.bfloat16).cuda()
        w0 = torch.from_numpy(p.w.view(np.int16)).view(torch.bfloat16).cuda()
        R = max(2, math.ceil(args.rotation_gib * 2**30 / (2 * N * K)))
        wp_dev[(N, K)] = [skg.skinny_gemm_pack_weight("bf16", w0) for _ in range(R)]
        w_dev[(N, K)] = [] if args.no_row_major else [w0] + [w0.clone() for _ in range(R - 1)]
        for M in Ms:
            y_dev[(M, N)] = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    log("inputs resident:", {f"{N}x{K}": len(wp_dev[(N, K)]) for N, K in shapes}, "copies per layout")

    stream = torch.cuda.current_stream()
    step_bytes = sum(alg_bytes(*c) for c in calls)
    # the split-K workspace of the device: the largest any call here needs
    # (the forms, mid-M and small-N reports register their own when larger)
    ensure_ws(skg, max(skg.skinny_gemm_workspace_bytes(op, *c) for c in calls for op in ("bf16", "bf16_packed")))

    def launcher(packed):
        def launch(c, copy):
            M, N, K = c
            if packed:
                ws = wp_dev[(N, K)]
                skg.skinny_gemm_bf16_packed(x_dev[K][:M], ws[copy % len(ws)], y=y_dev[(M, N)])
            else:
                ws = w_dev[(N, K)]
                skg.skinny_gemm_bf16(x_dev[K][:M], ws[copy % len(ws)], y=y_dev[(M, N)])
        return launch

    st = measure_step(args, torch, skg, calls, Ms, stream, launcher(True), "bf16_packed", step_bytes)
    row_major = None
    if not args.no_row_major:
        rm = measure_step(args, torch, skg, calls, Ms, stream, launcher(False), "bf16", step_bytes)
        row_major = {"value": round(rm["value"], 1), "ms_per_step": round(rm["ms_step"], 4),
                     "dominant_kernel": rm["dominant"], "avg_launch_us": round(rm["dom_us"], 3)}
        w_dev.clear()           # free the row-major copies
    launch, choice, dominant, dom_calls = st["launch"], st["choice"], st["dominant"], st["dom_calls"]
    rough_us, ms_step, dom_us, value = st["rough_us"], st["ms_step"], st["dom_us"], st["value"]

    if args.no_per_call:
        per_call_us = dict(rough_us)
        per_call_spread, per_call_eager = {}, {}
    else:
        # ------------------------------------------- per-call time (graph replay)
        per_call_us, per_call_spread, per_call_eager = {}, {}, {}
        for c in calls:
            M, N, K = c
            R = len(wp_dev[(N, K)])
            n = max(args.per_call_min, 2 * R)
            # eager: n launches from the host, no graph, between two events
            launch(c, 0)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for i in range(n):
                launch(c, i)
            b.record(stream)
            b.synchronize()
            per_call_eager[c] = a.elapsed_time(b) * 1e3 / n
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(n):
                    launch(c, i)
            g.replay()
            torch.cuda.synchronize()
            ts = []
            for _ in range(max(1, args.per_call_replays)):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                g.replay()
                b.record(stream)
                b.synchronize()
                ts.append(a.elapsed_time(b) * 1e3 / n)
            per_call_us[c] = statistics.median(ts)
            ts.sort()
            per_call_spread[c] = (ts[0], ts[min(len(ts) - 1, int(math.ceil(0.9 * len(ts))) - 1)])
            del g

    host_cost = None if args.no_per_call else measure_host_cost(torch, skg, x_dev, wp_dev, y_dev, stream)

    # ------------------------------------ achievable ceilings on this device
    # (profiling runs skip them, so that every dispatch profiled is the step's)
    ceil = None if args.no_per_call else measure_ceilings(args, torch, skg, shapes, wp_dev, stream)

    mid = None if (args.no_mid_m or ceil is None) else measure_mid_m(args, torch, skg, synth, shapes, wp_dev, stream, ceil)
    small_n = None if (args.no_small_n or ceil is None) else measure_small_n(args, torch, skg, synth, stream)
    forms = None if (args.no_forms or ceil is None) else measure_forms(args, torch, skg, synth, stream)

    # --------------------------- a copy of known size (counter calibration)
    src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst

    # ------------------------------------------------------------ report
    dom_bytes = sum(alg_bytes(*c) for c in dom_calls) / len(dom_calls)
    achieved = dom_bytes / (dom_us * 1e-6) / 1e9
    # the same launch mix at each shape's read ceiling (weight bytes read alone)
    achievable = None
    if ceil is not None:
        dom_ceil_us = sum(ceil["read"][(N, K)]["us"] for (_, N, K) in dom_calls) / len(dom_calls)
        achievable = dom_bytes / (dom_ceil_us * 1e-6) / 1e9
    code_hash = lib_code_hash()
    traffic = read_counters(dominant, code_hash)
    detail = {}
    compact = {}
    for M in (1, 8, 128):
        row, crow = {}, {}
        for (N, K) in shapes:
            c = (M, N, K)
            us = per_call_us[c]
            gbs = alg_bytes(*c) / (us * 1e-6) / 1e9
            tfl = 2 * M * N * K / (us * 1e-6) / 1e12
            row[f"{N}x{K}"] = {"us": round(us, 2), "GB/s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 3),
                               "mfma_frac": round(tfl / MFMA_BF16_PEAK_TFLOPS, 4), "variant": choice[c][0]}
            crow[f"{N}x{K}"] = [round(us, 2), round(gbs)]
            if c in per_call_spread:
                row[f"{N}x{K}"]["us_min"] = round(per_call_spread[c][0], 2)
                row[f"{N}x{K}"]["us_p90"] = round(per_call_spread[c][1], 2)
                row[f"{N}x{K}"]["eager_us"] = round(per_call_eager[c], 2)
            if ceil is not None:
                row[f"{N}x{K}"]["read_ceiling_frac"] = round(ceil["read"][(N, K)]["us"] / us, 3)
                row[f"{N}x{K}"]["mfma_ceiling_frac"] = round(tfl / ceil["mfma_bf16_tflops"], 4)
        detail[f"M={M}"] = row
        compact[str(M)] = crow
    all_calls = {f"{M}x{N}x{K}": round(per_call_us[(M, N, K)], 2) for (M, N, K) in calls}
    all_eager = {f"{M}x{N}x{K}": round(v, 2) for (M, N, K), v in per_call_eager.items()}

    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": round(traffic) if traffic is not None else None,
                "kernel": dominant, "launches_per_step": len(dom_calls), "avg_launch_us": round(dom_us, 3),
                "alg_bytes_per_launch": round(dom_bytes)}
    line = make_line(value, ms_step, args.steps, args.warmup, len(calls), roofline, compact)
    full = {
        **line,
        "config": {"workload": WORKLOAD, "weight_layout": "fragment-packed (skinny_gemm_pack_weight once per weight "
                                                          "copy, before timing; the same bytes)",
                   "calls_per_step": len(calls), "alg_bytes_per_step": step_bytes, "device": dev_name,
                   "table": skg.skinny_gemm_table_status()[1]},
        "row_major": row_major,
        "roofline": {**roofline, "code_hash": code_hash,
                     "achievable": None if achievable is None else
                     {"GB/s": round(achievable, 1), "frac": round(achieved / achievable, 4),
                      "basis": "the same launches at each shape's plain-read time of its weight "
                               "(skinny_gemm_calib_read, graph replay, best of 512..8192 workgroups in slices or "
                               "one sweep)"}},
        "ceilings": None if ceil is None else
        {"read": {f"{N}x{K}": v for (N, K), v in ceil["read"].items()},
         "mfma_bf16_tflops": round(ceil["mfma_bf16_tflops"], 1),
         "mfma_bf16_frac_of_peak": round(ceil["mfma_bf16_tflops"] / MFMA_BF16_PEAK_TFLOPS, 4)},
        "per_m": detail,
        "host_cost": host_cost,
        "mid_m": mid,
        "small_n": small_n,
        "forms": forms,
        "per_call_us": all_calls,
        "per_call_eager_us": all_eager or None,
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        cb = cpu_baseline(calls, host, args.cpu_seconds / 3)
        full["cpu_baseline"] = cb
        full["cpu_oracle_per_config"] = cpu_oracle_per_config(1.5)
        line["cpu_baseline"] = {k: cb[k] for k in ("value", "unit", "cores", "kind", "sample")}
    else:
        full["cpu_baseline"] = line["cpu_baseline"] = None
    if args.detail:
        os.makedirs(os.path.dirname(os.path.abspath(args.detail)), exist_ok=True)
        with open(args.detail, "w") as f:
            json.dump(full, f, indent=1)
    print(json.dumps(line, separators=(",", ":")), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

"""Summaries of rocprofv3 output for this library's kernels.

    python -m gemv_skinny_gemm_02_amd.profsum trace KERNEL_STATS.csv [--dispatches KERNEL_TRACE.csv] [--cmd CMD]
    python -m gemv_skinny_gemm_02_amd.profsum counters --fetch FETCH.csv --write WRITE.csv \
        --code-hash HASH [--cmd CMD]
    python -m gemv_skinny_gemm_02_amd.profsum mfma COUNTERS.csv [--cmd CMD]
    python -m gemv_skinny_gemm_02_amd.profsum pmc COUNTERS.csv [MORE.csv ...] [--cmd CMD]
    python -m gemv_skinny_gemm_02_amd.profsum form CALLS.json --trace KERNEL_TRACE.csv \
        [--fetch FETCH.csv --write WRITE.csv] [--pmc MORE.csv ...] [--cmd CMD]

`trace` prints the per-kernel call count and average/min/max duration from a
`--kernel-trace --stats` run.  `counters` turns two `--pmc FETCH_SIZE` and
`--pmc WRITE_SIZE` runs into KiB per dispatch for each kernel, and calibrates
both counters on the run's 256 MiB device-to-device copy (a copy of known size
reads and writes 262144 KiB): the factor is what the counter reads for that
copy divided by 262144.  HBM bytes per launch = FETCH/fetch_factor +
WRITE/write_factor, in KiB.  `mfma` summarises a `--pmc MfmaUtil
SQ_INSTS_VALU_MFMA_MOPS_BF16` run: MFMA utilisation and issued bf16 MFMA flops
per kernel.  `form` pairs the GEMM dispatches of a `bench.py --profile-form`
run, in launch order, with the call list that run wrote, and prints per call
shape (op, M, N, K, variant): the median device duration, the algorithmic
GB/s, and with the two counter runs the measured HBM bytes per launch and
their ratio to the algorithmic bytes, and the mean per launch of every
counter of any further `--pmc` runs (warm-up launches left out).
"""
from __future__ import annotations

import argparse
import csv
import statistics
import sys
from collections import defaultdict

COPY_KIB = 256 * 1024
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def trace_summary(path: str, cmd: str | None, dispatches: str | None = None) -> str:
    """Per kernel from the --stats file; with the per-dispatch trace file also
    the median device duration."""
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    med = {}
    if dispatches:
        durs = defaultdict(list)
        for r in csv.DictReader(open(dispatches)):
            durs[r["Kernel_Name"]].append(float(r["End_Timestamp"]) - float(r["Start_Timestamp"]))
        med = {k: statistics.median(v) for k, v in durs.items()}
    out = []
    if cmd:
        out.append(f"# command: {cmd}")
    out.append("# kernel | calls | avg_us | median_us | min_us | max_us | total_ms | percent")
    for r in rows:
        m = f"{med[r['Name']] / 1e3:.3f}" if r["Name"] in med else "nan"
        out.append(f"{r['Name']} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.3f} | {m} | {float(r['MinNs']) / 1e3:.3f} | "
                   f"{float(r['MaxNs']) / 1e3:.3f} | {float(r['TotalDurationNs']) / 1e6:.3f} | {float(r['Percentage']):.2f}")
    return "\n".join(out) + "\n"


def _per_kernel(path: str, counter: str):
    vals = defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            vals[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return vals


def _copy_factor(vals) -> float:
    cand = [v for v in vals.get(COPY_KERNEL, []) if 0.5 * COPY_KIB <= v <= 2.0 * COPY_KIB]
    if not cand:
        raise SystemExit("no 256 MiB copy dispatch found for calibration")
    return statistics.median(cand) / COPY_KIB


def counters_summary(fetch: str, write: str, code_hash: str, cmd: str | None) -> str:
    fv, wv = _per_kernel(fetch, "FETCH_SIZE"), _per_kernel(write, "WRITE_SIZE")
    ff, wf = _copy_factor(fv), _copy_factor(wv)
    out = []
    if cmd:
        out.append(f"# command: {cmd}")
    out.append("# FETCH_SIZE and WRITE_SIZE in KiB per dispatch (mean over the kernel's dispatches);")
    out.append("# HBM bytes per launch = (FETCH/copy_fetch_factor + WRITE/copy_write_factor) * 1024")
    out.append(f"code_hash={code_hash}")
    out.append(f"copy_fetch_factor={ff:.6f}")
    out.append(f"copy_write_factor={wf:.6f}")
    for name in sorted(set(fv) | set(wv)):
        if not name.startswith("void skg::"):
            continue
        f = statistics.fmean(fv[name]) if fv.get(name) else float("nan")
        w = statistics.fmean(wv[name]) if wv.get(name) else float("nan")
        out.append(f"kernel {name} | {f:.3f} | {w:.3f}")
    return "\n".join(out) + "\n"


def mfma_summary(path: str, cmd: str | None) -> str:
    """Per kernel: the mean MfmaUtil (MFMA-busy cycles over the dispatch's
    active cycles times the SIMD count, percent) and the bf16 MFMA flops it
    issued per dispatch (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512)."""
    util = _per_kernel(path, "MfmaUtil")
    mops = _per_kernel(path, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
    out = []
    if cmd:
        out.append(f"# command: {cmd}")
    out.append("# kernel | dispatches | MfmaUtil % (mean) | MfmaUtil % (max) | bf16 MFMA GFLOP issued per dispatch (mean)")
    for name in sorted(set(util) | set(mops)):
        if not name.startswith("void skg::"):
            continue
        u = util.get(name, [])
        m = mops.get(name, [])
        out.append(f"kernel {name} | {max(len(u), len(m))} | "
                   f"{statistics.fmean(u) if u else float('nan'):.2f} | {max(u) if u else float('nan'):.2f} | "
                   f"{statistics.fmean(m) * 512 / 1e9 if m else float('nan'):.4f}")
    return "\n".join(out) + "\n"


def pmc_summary(paths, cmd: str | None) -> str:
    """Per kernel, the mean per dispatch of every counter in one or more
    `--pmc` runs (one column per counter)."""
    vals = defaultdict(lambda: defaultdict(list))
    names = []
    for path in paths:
        for r in csv.DictReader(open(path)):
            c = r["Counter_Name"]
            if c not in names:
                names.append(c)
            vals[r["Kernel_Name"]][c].append(float(r["Counter_Value"]))
    out = []
    if cmd:
        out.append(f"# command: {cmd}")
    out.append("# kernel | dispatches | " + " | ".join(names) + "   (mean per dispatch)")
    for k in sorted(vals):
        if not k.startswith("void skg::"):
            continue
        n = max(len(v) for v in vals[k].values())
        cells = [f"{statistics.fmean(vals[k][c]):.6g}" if vals[k].get(c) else "nan" for c in names]
        out.append(f"kernel {k} | {n} | " + " | ".join(cells))
    return "\n".join(out) + "\n"


GEMM_KERNELS = ("void skg::gemv_kernel", "void skg::tile_kernel", "void skg::tlds_kernel", "void skg::mt_kernel",
                "void skg::pg_kernel")


def _gemm_dispatches(path: str, counter: str | None = None):
    """The GEMM dispatches of one run in dispatch order: (kernel, value), the
    value being the duration in ns (trace file) or the counter (pmc file)."""
    rows = []
    for r in csv.DictReader(open(path)):
        if not r["Kernel_Name"].startswith(GEMM_KERNELS):
            continue
        if counter is None:
            v = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
        elif r["Counter_Name"] == counter:
            v = float(r["Counter_Value"])
        else:
            continue
        rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], v))
    rows.sort()
    return [(k, v) for _, k, v in rows]


def _pair(launches, disp, what):
    if len(disp) != len(launches):
        raise SystemExit(f"{what}: {len(disp)} GEMM dispatches for {len(launches)} calls")
    return list(zip(launches, disp))


# Ratios printed beside the raw counters when a run holds what they need.
DERIVED_NEEDS = {
    "wait_frac": ("SQ_WAIT_ANY", "SQ_WAVE_CYCLES"),
    "lds_conflict_frac": ("SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE"),
    "l2_read_latency_cyc": ("TCP_TCC_READ_REQ_LATENCY_sum", "TCP_TCC_READ_REQ_sum"),
    "ta_units_stalled": ("TA_ADDR_STALLED_BY_TC_CYCLES_sum", "TA_BUSY_avr"),
}
DERIVED_DOC = {
    "wait_frac": "SQ_WAIT_ANY / SQ_WAVE_CYCLES: share of wave cycles spent waiting on a counter (memory, LDS)",
    "lds_conflict_frac": "SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE: share of LDS cycles lost to bank conflicts",
    "l2_read_latency_cyc": "TCP_TCC_READ_REQ_LATENCY_sum / TCP_TCC_READ_REQ_sum: mean L1->L2 read latency, cycles",
    "ta_units_stalled": "TA_ADDR_STALLED_BY_TC_CYCLES_sum / TA_BUSY_avr: address-stall cycles (waiting on the "
                        "vector L1) summed over the TA units per busy cycle of the average unit, i.e. how many "
                        "units are stalled at once on average",
}
DERIVED = [
    ("wait_frac", lambda v: v["SQ_WAIT_ANY"] / v["SQ_WAVE_CYCLES"]),
    ("lds_conflict_frac", lambda v: v["SQ_LDS_BANK_CONFLICT"] / v["SQ_LDS_IDX_ACTIVE"]),
    ("l2_read_latency_cyc", lambda v: v["TCP_TCC_READ_REQ_LATENCY_sum"] / v["TCP_TCC_READ_REQ_sum"]),
    ("ta_units_stalled", lambda v: v["TA_ADDR_STALLED_BY_TC_CYCLES_sum"] / v["TA_BUSY_avr"]),
]


def form_summary(calls: str, trace: str, fetch: str | None, write: str | None, cmd: str | None,
                 pmc=()) -> str:
    import json
    info = json.load(open(calls))
    launches = info["launches"]
    t = _pair(launches, _gemm_dispatches(trace), "trace")
    groups = defaultdict(lambda: defaultdict(list))
    order = []
    for c, (k, ns) in t:
        key = (c["op"], c["M"], c["N"], c["K"], c["variant"], k, c["alg_bytes"])
        if key not in order:
            order.append(key)
        if not c["warm"]:
            groups[key]["ns"].append(ns)
    ff = wf = None
    if fetch and write:
        ff = _copy_factor(_per_kernel(fetch, "FETCH_SIZE"))
        wf = _copy_factor(_per_kernel(write, "WRITE_SIZE"))
        for col, path, ctr in (("f", fetch, "FETCH_SIZE"), ("w", write, "WRITE_SIZE")):
            for c, (k, v) in _pair(launches, _gemm_dispatches(path, ctr), ctr):
                if not c["warm"]:
                    groups[(c["op"], c["M"], c["N"], c["K"], c["variant"], k, c["alg_bytes"])][col].append(v)
    extra = []
    for path in pmc:
        names = []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] not in names:
                names.append(r["Counter_Name"])
        for ctr in names:
            extra.append(ctr)
            for c, (k, v) in _pair(launches, _gemm_dispatches(path, ctr), ctr):
                if not c["warm"]:
                    groups[(c["op"], c["M"], c["N"], c["K"], c["variant"], k, c["alg_bytes"])][ctr].append(v)
    derived = [(name, f) for name, f in DERIVED if all(c in extra for c in DERIVED_NEEDS[name])]
    out = []
    if cmd:
        out.append(f"# command: {cmd}")
    for name, _ in derived:
        out.append(f"# {name} = {DERIVED_DOC[name]}")
    out.append(f"# form {info['form']}: {len(launches)} calls in launch order, paired one to one with the GEMM "
               "dispatches; warm-up launches dropped")
    if ff is not None:
        out.append(f"# copy_fetch_factor={ff:.6f} copy_write_factor={wf:.6f} (the run's 256 MiB device copy); "
                   "hbm_MB = (FETCH/fetch_factor + WRITE/write_factor) KiB per launch")
    out.append("# op | M | N | K | variant | launches | median_us | alg_MB | alg_GB/s | hbm_MB | hbm/alg | "
               + "".join(f"{e} | " for e in extra) + "".join(f"{n} | " for n, _ in derived) + "kernel"
               + ("   (counters: mean per launch)" if extra else ""))
    for key in order:
        op, M, N, K, var, k, nb = key
        g = groups[key]
        if not g["ns"]:
            continue
        us = statistics.median(g["ns"]) / 1e3
        line = f"{op} | {M} | {N} | {K} | {var} | {len(g['ns'])} | {us:.3f} | {nb / 1e6:.3f} | {nb / (us * 1e3):.1f}"
        if ff is not None and g["f"] and g["w"]:
            hb = (statistics.fmean(g["f"]) / ff + statistics.fmean(g["w"]) / wf) * 1024
            line += f" | {hb / 1e6:.3f} | {hb / nb:.3f}"
        else:
            line += " | nan | nan"
        for e in extra:
            line += f" | {statistics.fmean(g[e]):.6g}" if g[e] else " | nan"
        for _, fn in derived:
            try:
                line += f" | {fn({c: statistics.fmean(g[c]) for c in extra if g[c]}):.3f}"
            except (KeyError, ZeroDivisionError):
                line += " | nan"
        out.append(line + f" | {k}")
    return "\n".join(out) + "\n"


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="mode", required=True)
    t = sub.add_parser("trace")
    t.add_argument("stats")
    t.add_argument("--dispatches", help="the per-dispatch kernel trace csv, for the median")
    t.add_argument("--cmd")
    c = sub.add_parser("counters")
    c.add_argument("--fetch", required=True)
    c.add_argument("--write", required=True)
    c.add_argument("--code-hash", required=True)
    c.add_argument("--cmd")
    q = sub.add_parser("pmc")
    q.add_argument("counters", nargs="+")
    q.add_argument("--cmd")
    m = sub.add_parser("mfma")
    m.add_argument("counters")
    m.add_argument("--cmd")
    f = sub.add_parser("form")
    f.add_argument("calls")
    f.add_argument("--trace", required=True, help="the per-dispatch kernel trace csv")
    f.add_argument("--fetch")
    f.add_argument("--write")
    f.add_argument("--pmc", action="append", default=[], help="a further counter run (repeatable)")
    f.add_argument("--cmd")
    a = ap.parse_args(argv)
    if a.mode == "form":
        sys.stdout.write(form_summary(a.calls, a.trace, a.fetch, a.write, a.cmd, a.pmc))
    elif a.mode == "trace":
        sys.stdout.write(trace_summary(a.stats, a.cmd, a.dispatches))
    elif a.mode == "pmc":
        sys.stdout.write(pmc_summary(a.counters, a.cmd))
    elif a.mode == "mfma":
        sys.stdout.write(mfma_summary(a.counters, a.cmd))
    else:
        sys.stdout.write(counters_summary(a.fetch, a.write, a.code_hash, a.cmd))
    return 0


if __name__ == "__main__":
    sys.exit(main())

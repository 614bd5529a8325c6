"""Measuring tuner and promotion for the per-device dispatch table.

    python -m gemv_skinny_gemm_02_amd.tuner tune  --store STORE.jsonl [--ops bf16,gated,...] [--rows decode|mid|all] [--quick]
    python -m gemv_skinny_gemm_02_amd.tuner promote --store STORE.jsonl --out TABLE.json [--merge OLD_TABLE.json]
    python -m gemv_skinny_gemm_02_amd.tuner check [--table TABLE.json]

`tune` runs on the GPU.  For every key (op, rows bucket, N, K) of the workload
set it runs every compiled variant that can serve the bucket, checks its
output against the built-in default's output at the parity bar (a variant that
disagrees is recorded as failed and never promoted), and times it the way the
benchmark does: weight copies rotated past the Infinity Cache, launches
replayed from a HIP graph, the median of several replays.  Every measurement is
appended to the JSONL store with the device identity; a rerun skips
(identity, key, variant) triples already stored, so the store is also the
checkpoint.

`promote` is a pure function of the store.  For each key the built-in default
is the incumbent; a different variant is chosen only when its time is at least
2 % below the default's (the promote threshold of mstar PR #1104, "What
changed"; candidates are measured against the incumbent's own entry point as
in Decode optimization round 3, "Rejected paths", and Strata PR #1297, item 4,
the true-default baseline).  The table
keeps every candidate's time beside the choice, so moving a size is a one-word
edit, and `check` re-derives every choice from the times the table carries.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

import numpy as np

KEEP_GAIN = 0.02          # a non-default variant must be >= 2 % faster
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------ workload keys
def workload_keys(ops, rows="decode"):
    """(op, M, N, K) for every configured workload shape.  rows: "decode" (the
    decode rows of each form), "mid" (the mid-M rows: bf16 sweep shapes and the
    A8W8 shapes),
    "smalln" (the small-N bf16 shapes) or "all"."""
    sys.path.insert(0, ROOT)
    import synth
    keys = []
    if rows in ("mid", "all"):
        for op in ("bf16", "bf16_packed"):
            if op in ops:
                keys += [(op, M, N, K) for (N, K) in synth.SWEEP_NK for M in synth.MID_M]
        for op in ("a8w8_block", "a8w8_block_packed"):
            if op in ops:
                keys += [(op, M, N, K) for (N, K) in synth.A8W8_NK for M in synth.MID_M]
    if rows in ("smalln", "all"):
        for op in ("bf16", "bf16_packed"):
            if op in ops:
                keys += [(op, M, N, K) for (N, K) in synth.SMALLN_NK for M in synth.SMALLN_M]
    if rows in ("mid", "smalln"):
        return keys
    if "bf16" in ops:
        keys += [("bf16", M, N, K) for (N, K) in synth.SWEEP_NK for M in synth.SWEEP_M]
    if "gated" in ops:
        N, K = synth.GATED_NK
        keys += [("gated", M, N, K) for M in synth.GATED_M]
    if "fp8_tensor" in ops:
        N, K = synth.HEAD_NK
        keys += [("fp8_tensor", M, N, K) for M in synth.HEAD_M]
    if "a8w8_block" in ops:
        keys += [("a8w8_block", M, N, K) for (N, K) in synth.A8W8_NK for M in synth.A8W8_M]
    if "a8w8_quant" in ops:
        keys += [("a8w8_quant", M, N, K) for (N, K) in synth.A8W8_NK for M in synth.A8W8_M]
    # the packed forms run on the same shapes as their row-major forms
    for op in [o for o in ops if o.endswith("_packed")]:
        keys += [(op, M, N, K) for (_, M, N, K) in workload_keys([op[:-len("_packed")]])]
    return keys


def base_op(op):
    """The row-major form of an op name."""
    return op[:-len("_packed")] if op.endswith("_packed") else op


def bucket_of(M):
    from gemv_skinny_gemm_02_amd import BUCKETS
    for b in BUCKETS:
        if M <= b:
            return b
    return 0


def alg_bytes(op, M, N, K):
    op = base_op(op)
    if op == "bf16":
        return 2 * N * K + 2 * M * K + 2 * M * N
    if op == "gated":
        return 4 * N * K + 2 * M * K + 2 * M * N
    if op == "fp8_tensor":
        return N * K + 2 * M * K + 2 * M * N + 4
    kb, nb = -(-K // 128), -(-N // 128)
    if op == "a8w8_quant":                       # bf16 x in, no x scales read
        return N * K + 2 * M * K + 4 * nb * kb + 2 * M * N
    return N * K + M * K + 4 * M * kb + 4 * nb * kb + 2 * M * N


# ------------------------------------------------------------------- store
def read_store(path):
    out = []
    if os.path.exists(path):
        with open(path) as f:
            for line in f:
                line = line.strip()
                if line:
                    out.append(json.loads(line))
    return out


def _close_bf16(a, b):
    """Parity bar between two bf16 results of the same problem (both rounded):
    max |a-b| <= 2^-7 max|b| and relative Frobenius <= 5e-3."""
    import torch
    a = a.float()
    b = b.float()
    if not torch.isfinite(a).all():
        return False
    mx = b.abs().max().item()
    d = (a - b).abs().max().item()
    fro = (torch.linalg.norm(a - b) / max(torch.linalg.norm(b).item(), 1e-30)).item()
    return d <= 2.0 ** -7 * mx and fro <= 5e-3


def tune(store, ops, quick=False, rotation_gib=1.0, replays=5, only_m=None, rows="decode"):
    import torch

    import gemv_skinny_gemm_02_amd as skg
    import synth

    torch.cuda.set_device(0)
    skg.load()
    # split-K partials of up to 256 MiB (a candidate that needs more is
    # recorded as refused), plus the arrival counters
    skg.skinny_gemm_set_device_workspace((256 << 20) + (256 << 10))
    ident = skg.skinny_gemm_identity()
    # measured triples are skipped on a rerun; a recorded failure is retried
    done = {(r["identity"], r["op"], r["rows"], r["N"], r["K"], r["variant"]) for r in read_store(store)
            if "us" in r}
    keys = workload_keys(ops, rows)
    if only_m:
        keys = [k for k in keys if k[1] in only_m]
    stream = torch.cuda.current_stream()
    make = {"bf16": synth.make_bf16, "gated": synth.make_gated, "fp8_tensor": synth.make_fp8_tensor,
            "a8w8_block": synth.make_a8w8_block, "a8w8_quant": synth.make_a8w8_quant}
    ops = list(ops)
    cache = {}
    with open(store, "a") as fout:
        for (op, M, N, K) in keys:
            b = bucket_of(M)
            names = skg.variants(op)
            cands = [i for i, n in enumerate(names) if skg.skinny_gemm_variant_supports(op, i, M)]
            todo = [i for i in cands if (ident, op, b, N, K, names[i]) not in done]
            if not todo:
                continue
            shape_key = (op, N, K)
            bop = base_op(op)
            if shape_key not in cache:
                cache.clear()
                torch.cuda.empty_cache()
                p = make[bop](max(m for (o, m, n, k) in keys if (o, n, k) == shape_key), N, K, seed=0)
                if bop in ("bf16", "gated"):
                    x = torch.from_numpy(p.x.view(np.int16)).view(torch.bfloat16).cuda()
                    w0 = torch.from_numpy(p.w.view(np.int16)).view(torch.bfloat16).cuda()
                else:
                    x = (torch.from_numpy(p.x.view(np.int16)).view(torch.bfloat16) if bop in ("fp8_tensor", "a8w8_quant")
                         else torch.from_numpy(p.x).view(torch.float8_e4m3fn)).cuda()
                    w0 = torch.from_numpy(p.w).view(torch.float8_e4m3fn).cuda()
                s0 = torch.from_numpy(p.s0).cuda() if p.s0 is not None else None
                s1 = torch.from_numpy(p.s1).cuda() if p.s1 is not None else None
                R = max(2, math.ceil(rotation_gib * 2**30 / (w0.numel() * w0.element_size())))
                free, _ = torch.cuda.mem_get_info()
                R = max(1, min(R, int(0.6 * free // (w0.numel() * w0.element_size()))))
                if op != bop:      # packed copies, each packed from the same weight
                    ws = [skg.skinny_gemm_pack_weight(bop, w0) for _ in range(R)]
                    del w0
                else:
                    ws = [w0] + [w0.clone() for _ in range(R - 1)]
                cache[shape_key] = (x, ws, s0, s1)
            x, ws, s0, s1 = cache[shape_key]
            xm = x[:M]
            s0m = s0[:M] if (bop == "a8w8_block" and s0 is not None) else s0
            y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
            # the true default: what dispatch runs with no table
            default_name = skg.skinny_gemm_query(op, M, N, K)[0] if not skg.skinny_gemm_table_status()[0] else None
            if default_name is None:
                raise SystemExit("tune with no table engaged (SKINNY_GEMM_TABLE pointing at a missing file)")
            ref = skg.skinny_gemm_run_variant(op, default_name, xm, ws[0], s0m, s1).clone()
            n = max(16 if quick else 64, 2 * len(ws))
            for i in todo:
                name = names[i]
                rec = {"identity": ident, "op": op, "rows": b, "M": M, "N": N, "K": K, "variant": name,
                       "default": default_name, "time": time.time()}
                try:
                    out = skg.skinny_gemm_run_variant(op, i, xm, ws[0], s0m, s1, y=y)
                    torch.cuda.synchronize()
                    rec["parity_vs_default"] = bool(_close_bf16(out, ref))
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g):
                        for j in range(n):
                            skg.skinny_gemm_run_variant(op, i, xm, ws[j % len(ws)], s0m, s1, y=y)
                    g.replay()
                    torch.cuda.synchronize()
                    ts = []
                    for _ in range(2 if quick else replays):
                        a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                        a.record(stream)
                        g.replay()
                        e.record(stream)
                        e.synchronize()
                        ts.append(a.elapsed_time(e) * 1e3 / n)
                    del g
                    rec["us"] = statistics.median(ts)
                    rec["samples_us"] = [round(t, 4) for t in ts]
                    rec["gbs"] = alg_bytes(op, M, N, K) / (rec["us"] * 1e-6) / 1e9
                except Exception as ex:  # a refused launch is recorded, not fatal
                    rec["error"] = str(ex)
                fout.write(json.dumps(rec) + "\n")
                fout.flush()
                log(f"{op} M={M} N={N} K={K} {name}: {rec.get('us', float('nan')):.2f} us "
                    f"{rec.get('gbs', 0):.0f} GB/s parity={rec.get('parity_vs_default')}")
    return 0


def choose(default, times):
    """The promotion rule: `times` maps each measured variant to its µs.  The
    fastest variant (ties: the first name) replaces the built-in default only
    when it is at least KEEP_GAIN faster; a default that was not measured
    gives way to the fastest."""
    best = min(sorted(times), key=lambda v: times[v])
    if default in times and best != default and times[best] > (1.0 - KEEP_GAIN) * times[default]:
        return default
    return best


def check(table_path):
    """Re-derive every entry's choice from the candidate times the table
    carries (the store's per-variant medians) with the promotion rule; returns
    the entries whose stored choice differs (an empty list: the table is what
    promotion of its own measurements gives)."""
    with open(table_path) as f:
        t = json.load(f)
    bad = []
    for e in t["entries"]:
        times = {v: c["us"] for v, c in e.get("candidates", {}).items()}
        if not times:
            bad.append((e["op"], e["rows"], e["N"], e["K"], "no candidates"))
            continue
        want = choose(e["default"], times)
        if want != e["choice"] or abs(times[e["choice"]] - e["us"]) > 1e-9:
            bad.append((e["op"], e["rows"], e["N"], e["K"], e["choice"], want))
    return bad


def promote(store, out, identity=None, merge=None):
    """Write the table from the store (pure function of the store).  merge: an
    existing table of the same identity whose entries for keys the store does
    not measure are kept as they are."""
    recs = [r for r in read_store(store) if "us" in r and r.get("parity_vs_default")]
    if not recs:
        raise SystemExit("store holds no usable measurements")
    idents = sorted({r["identity"] for r in recs})
    ident = identity or idents[-1]
    recs = [r for r in recs if r["identity"] == ident]
    by_key = {}
    for r in recs:
        k = (r["op"], r["rows"], r["N"], r["K"])
        # several M can share a bucket; keep the largest M's measurement (the bucket's worst case)
        slot = by_key.setdefault(k, {})
        prev = slot.get(r["variant"])
        if prev is None or r["M"] > prev["M"] or (r["M"] == prev["M"] and r["time"] > prev["time"]):
            slot[r["variant"]] = r
    entries = []
    order = {"bf16": 0, "gated": 1, "fp8_tensor": 2, "a8w8_block": 3, "a8w8_quant": 4,
             "bf16_packed": 5, "gated_packed": 6, "fp8_tensor_packed": 7, "a8w8_block_packed": 8,
             "a8w8_quant_packed": 9}
    for k in sorted(by_key, key=lambda k: (order[k[0]], k[2], k[3], k[1])):
        slot = by_key[k]
        default = next(iter(slot.values()))["default"]
        cands = sorted(slot.values(), key=lambda r: (r["us"], r["variant"]))
        # the rule sees the times the table stores (rounded to the ns), so that
        # `check` re-derives exactly this choice
        choice = choose(default, {r["variant"]: round(r["us"], 3) for r in cands})
        entries.append({"op": k[0], "rows": k[1], "N": k[2], "K": k[3], "choice": choice, "default": default,
                        "measured_M": slot[choice]["M"], "us": round(slot[choice]["us"], 3),
                        "candidates": {r["variant"]: {"us": round(r["us"], 3)} for r in cands}})
    idd = dict(kv.split("=", 1) for kv in ident.split(";"))
    if merge:
        with open(merge) as f:
            old = json.load(f)
        if old.get("identity") != idd:
            raise SystemExit(f"{merge}: identity {old.get('identity')} differs from the store's {idd}")
        have = {(e["op"], e["rows"], e["N"], e["K"]) for e in entries}
        kept = [e for e in old["entries"] if (e["op"], e["rows"], e["N"], e["K"]) not in have]
        entries = sorted(kept + entries, key=lambda e: (order[e["op"]], e["N"], e["K"], e["rows"]))
        log(f"merged: {len(kept)} entries kept from {merge}")
    table = {"format": "skinny_gemm_table", "version": 1, "identity": idd,
             "rule": f"non-default choice only at >= {KEEP_GAIN:.0%} gain over the built-in default",
             "entries": entries}
    os.makedirs(os.path.dirname(os.path.abspath(out)), exist_ok=True)
    with open(out, "w") as f:
        json.dump(table, f, indent=1)
        f.write("\n")
    moved = sum(e["choice"] != e["default"] for e in entries)
    log(f"wrote {out}: {len(entries)} entries, {moved} away from the default")
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="mode", required=True)
    t = sub.add_parser("tune")
    t.add_argument("--store", required=True)
    t.add_argument("--ops", default="bf16,gated,fp8_tensor,a8w8_block,a8w8_quant,bf16_packed,gated_packed,"
                                    "fp8_tensor_packed,a8w8_block_packed,a8w8_quant_packed")
    t.add_argument("--quick", action="store_true")
    t.add_argument("--rotation-gib", type=float, default=1.0)
    t.add_argument("--only-m", default="")
    t.add_argument("--rows", default="decode", choices=("decode", "mid", "smalln", "all"))
    p = sub.add_parser("promote")
    p.add_argument("--store", required=True)
    p.add_argument("--out", required=True)
    p.add_argument("--identity", default=None)
    p.add_argument("--merge", default=None, help="existing table whose other entries are kept")
    c = sub.add_parser("check")
    c.add_argument("--table", default=None, help="table to check (default: the installed gfx950 table)")
    a = ap.parse_args(argv)
    if a.mode == "check":
        path = a.table or os.path.join(ROOT, "gemv_skinny_gemm_02_amd", "configs", "gfx950", "skinny_gemm.json")
        bad = check(path)
        for b in bad:
            log("differs:", b)
        log(f"{path}: {'every choice follows from its candidate times' if not bad else f'{len(bad)} entries differ'}")
        return 1 if bad else 0
    if a.mode == "tune":
        os.environ.setdefault("SKINNY_GEMM_TABLE", "/nonexistent/skinny_gemm.json")  # measure the true defaults
        only = [int(v) for v in a.only_m.split(",") if v]
        return tune(a.store, a.ops.split(","), a.quick, a.rotation_gib, only_m=only, rows=a.rows)
    return promote(a.store, a.out, a.identity, a.merge)


if __name__ == "__main__":
    sys.exit(main())

"""Host logic of bench.py: the kernel symbol a variant runs as, and the
traffic lookup in a counter summary (no GPU)."""
import os

import pytest

import bench
import gemv_skinny_gemm_02_amd as skg


@pytest.mark.parametrize("variant,M,symbol", [
    ("gemv_r2_k4_p1", 1, "void skg::gemv_kernel<0, 1, 2, 4, 1>(skg::Args)"),
    ("gemv_r4_k1_p2", 7, "void skg::gemv_kernel<0, 8, 4, 1, 2>(skg::Args)"),
    ("tile_f1_k4_p4", 24, "void skg::tile_kernel<0, 2, 1, 4, 4>(skg::Args)"),
    ("tlds_f1_s4_p4", 16, "void skg::tlds_kernel<0, 1, 1, 4, 4, 4, 1, 0>(skg::Args)"),
    ("tlds_f1_s4_p4", 128, "void skg::tlds_kernel<0, 8, 1, 4, 4, 4, 1, 0>(skg::Args)"),
    ("tlds_f1_s4_p4_m2", 128, "void skg::tlds_kernel<0, 2, 1, 4, 4, 4, 1, 0>(skg::Args)"),
    ("tlds_w8_f1_s4_p4_m4", 96, "void skg::tlds_kernel<0, 4, 1, 4, 4, 8, 1, 0>(skg::Args)"),
    ("tlds_k4_f1_s1_p4_m1", 64, "void skg::tlds_kernel<0, 1, 1, 1, 4, 4, 4, 0>(skg::Args)"),
    ("tlds_w8_k8_f1_s1_p2_m1", 128, "void skg::tlds_kernel<0, 1, 1, 1, 2, 8, 8, 0>(skg::Args)"),
    ("tlds_f1_s4_p4", 40, "void skg::tlds_kernel<0, 4, 1, 4, 4, 4, 1, 0>(skg::Args)"),   # 3 fragments -> the 4 build
    ("tlds_d_k4_f1_s1_p4_m1", 4, "void skg::tlds_kernel<0, 1, 1, 1, 4, 4, 4, 1>(skg::Args)"),
    ("tlds_d_w8_k8_f1_s1_p4_m2", 32, "void skg::tlds_kernel<0, 2, 1, 1, 4, 8, 8, 1>(skg::Args)"),
    ("tlds_x_w8_k2_f2_s4_p2_m4", 128, "void skg::tlds_kernel<0, 4, 2, 4, 2, 8, 2, 2>(skg::Args)"),
    ("mt_m4_f2_a2_b4_s2_p3", 512, "void skg::mt_kernel<0, 4, 2, 2, 4, 2, 3>(skg::Args)"),   # any M: one build
])
def test_kernel_symbol(variant, M, symbol):
    assert bench.kernel_symbol(variant, M) == symbol


def test_every_variant_name_parses():
    for op in ("bf16", "bf16_packed", "a8w8_block_packed"):
        for i, name in enumerate(skg.variants(op)):
            for M in (1, 16, 128):
                if not skg.skinny_gemm_variant_supports(op, i, M):
                    continue
                sym = bench.kernel_symbol(name, M, skg.OPS[op])
                assert sym.startswith("void skg::") and sym.endswith("(skg::Args)")
                if name.startswith("mt_"):
                    v = [int(p[1:]) for p in name.split("_")[1:]]
                    assert sym == f"void skg::mt_kernel<{skg.OPS[op]}, {', '.join(map(str, v))}>(skg::Args)", (name, sym)
                if name.startswith("tlds"):
                    xd = 1 if name.startswith("tlds_d_") else (2 if name.startswith("tlds_x_") else 0)
                    assert sym.endswith(f", {xd}>(skg::Args)"), (name, sym)


def test_read_counters(tmp_path, monkeypatch):
    os.makedirs(tmp_path / "profiles")
    (tmp_path / "profiles" / "bf16_sweep_counters.txt").write_text(
        "# comment\ncode_hash=abc\ncopy_fetch_factor=0.5\ncopy_write_factor=1.0\n"
        "kernel void skg::k<0>(skg::Args) | 100.0 | 10.0\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    # HBM bytes = (FETCH / fetch factor + WRITE / write factor) KiB
    assert bench.read_counters("void skg::k<0>(skg::Args)", "abc") == (100.0 / 0.5 + 10.0) * 1024
    assert bench.read_counters("void skg::k<1>(skg::Args)", "abc") is None     # kernel not profiled
    assert bench.read_counters("void skg::k<0>(skg::Args)", "other") is None   # sources changed since


@pytest.mark.parametrize("form", ["bf16", "gated", "fp8_tensor", "a8w8_block", "a8w8_quant"])
def test_alg_bytes_agree(form):
    """The bench's algorithmic bytes per call are the tuner's, for every form,
    and the weight term dominates as the formulas say (W once; x, scales and y
    once each)."""
    from gemv_skinny_gemm_02_amd import tuner
    for (M, N, K) in [(1, 4096, 4096), (64, 8192, 4096), (3, 248320, 4096), (16, 32768, 1024), (5, 257, 1040)]:
        want = tuner.alg_bytes(form, M, N, K)
        got = bench.alg_bytes(M, N, K) if form == "bf16" else bench.form_alg_bytes(form, M, N, K)
        assert got == want, (form, M, N, K)
    # the weight alone, in bytes: 2NK (bf16), 4NK (gate and up), NK (fp8)
    wb = {"bf16": 2, "gated": 4, "fp8_tensor": 1, "a8w8_block": 1, "a8w8_quant": 1}[form]
    assert tuner.alg_bytes(form, 1, 4096, 4096) - wb * 4096 * 4096 < 0.01 * wb * 4096 * 4096


def test_bench_gpus_flag_refuses_more_than_one():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_printed_line_is_short():
    """The line the benchmark prints holds the headline fields, the roofline
    and the CPU baseline, and stays under 2 KB, so that a reader of the last
    few KB of the output gets all of it."""
    import json
    shapes = ["4096x4096", "6144x4096", "4096x12288", "2048x2048", "1024x1024"]
    per_m = {str(M): {s: [123.45, 7654] for s in shapes} for M in (1, 8, 128)}
    roofline = {"bound": "hbm", "achieved": 4486.3, "peak": 8000.0, "unit": "GB/s", "frac": 0.5608,
                "traffic": 35190123, "kernel": "void skg::tlds_kernel<5, 1, 1, 1, 4, 4, 4, 1>(skg::Args)",
                "launches_per_step": 26, "avg_launch_us": 7.812, "alg_bytes_per_launch": 34830494}
    cpu = {"value": 1.3908, "unit": "GB/s", "cores": 16, "kind": "oracle",
           "sample": "median of 3 runs of 5 s, each the step's 65 calls in order (170-180 calls), "
                     "oracle.linear_bf16 in float64 on 16 BLAS threads of 128 host cores"}
    line = bench.make_line(3859.2, 0.6654, 20, 5, 65, roofline, per_m, cpu)
    text = json.dumps(line, separators=(",", ":"))
    assert len(text) < 2048, len(text)
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
              "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert k in line
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in line["roofline"]
    assert line["metric"] == "achieved HBM GB/s and \u00b5s/call at M=1/8/128; fraction of MI355X roofline"


def test_profsum_form_pairs_dispatches_with_calls(tmp_path):
    """The form summary pairs GEMM dispatches with the call list in dispatch
    order, skips non-GEMM kernels and warm-up launches, and calibrates the
    counters on the 256 MiB copy."""
    import csv
    import json

    from gemv_skinny_gemm_02_amd import profsum

    gemm = "void skg::tlds_kernel<5, 1, 1, 1, 4, 4, 4, 0>(skg::Args)"
    other = "void skg::(anonymous namespace)::pack_kernel<false>(char const*)"
    calls = [{"op": "bf16_packed", "M": 8, "N": 1024, "K": 1024, "alg_bytes": 2_000_000, "warm": w,
              "variant": "tlds_f1_s1_p4_m4"} for w in (True, False, False)]
    (tmp_path / "calls.json").write_text(json.dumps({"form": "bf16", "launches": calls}))
    # dispatch ids out of file order on purpose; a pack dispatch in between
    trace = [(3, gemm, 0, 1000), (1, gemm, 0, 9000), (2, other, 0, 5), (4, gemm, 0, 3000)]
    with open(tmp_path / "trace.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writerows(trace)
    for name, ctr, copy_v, v in (("fetch", "FETCH_SIZE", 131072.0, 1000.0), ("write", "WRITE_SIZE", 262144.0, 16.0)):
        with open(tmp_path / f"{name}.csv", "w", newline="") as f:
            w = csv.writer(f)
            w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
            w.writerow([1, gemm, ctr, 99999.0])
            w.writerow([3, gemm, ctr, v])
            w.writerow([4, gemm, ctr, v])
            w.writerow([5, profsum.COPY_KERNEL, ctr, copy_v])
    out = profsum.form_summary(str(tmp_path / "calls.json"), str(tmp_path / "trace.csv"),
                               str(tmp_path / "fetch.csv"), str(tmp_path / "write.csv"), "cmd")
    row = [l for l in out.splitlines() if l.startswith("bf16_packed")]
    assert len(row) == 1
    cells = [c.strip() for c in row[0].split("|")]
    assert cells[5] == "2"                      # two timed launches, the warm one dropped
    assert cells[6] == "2.000"                  # median of 1 us and 3 us
    assert cells[8] == "1000.0"                 # 2 MB / 2 us
    assert abs(float(cells[9]) - (1000 / 0.5 + 16) * 1024 / 1e6) < 1e-3
    with pytest.raises(SystemExit):             # a count mismatch is refused, not paired loosely
        profsum._pair(calls, [("k", 1.0)], "trace")

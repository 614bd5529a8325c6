"""Every entry of the installed dispatch table, served from a graph replay,
against the CPU oracle (mstar PR #1104, "Verification": every kernel the table
holds is checked against the parity bar from a graph replay).

For each (op, N, K) of the table the inputs are drawn once at the largest rows
bucket of that shape, and each entry runs at its bucket's M: row m of the
linear depends on row m of x only, so the oracle's result sliced to the first
M rows is the reference.  Every output is compared, except on the 248320-row
vocabulary head: one seeded column in every 16-row block.
"""
import json
from collections import defaultdict

import numpy as np
import pytest
import torch

import gemv_skinny_gemm_02_amd as skg
import oracle
import synth
from gpu_util import assert_parity, dev_bf16, dev_f32, dev_fp8, ensure_workspace, host_bits, say
from test_gpu_parity import head_cols

pytestmark = pytest.mark.gpu

MAKE = {"bf16": synth.make_bf16, "gated": synth.make_gated, "fp8_tensor": synth.make_fp8_tensor,
        "a8w8_block": synth.make_a8w8_block, "a8w8_quant": synth.make_a8w8_quant}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    skg.load()
    ensure_workspace()
    skg.skinny_gemm_query("bf16", 1, 4096, 4096)          # loads the installed table
    engaged, status = skg.skinny_gemm_table_status()
    say("table:", status)
    assert engaged, f"the installed table does not engage on this device: {status}"


def _entries(op):
    with open(skg.default_table_path()) as f:
        t = json.load(f)
    by_shape = defaultdict(list)
    for e in t["entries"]:
        if e["op"] == op:
            by_shape[(e["N"], e["K"])].append(e)
    return by_shape


def _call(op, x, w, s0, s1, y):
    base = op[:-len("_packed")] if op.endswith("_packed") else op
    fn = getattr(skg, "skinny_gemm_" + {"a8w8_block": "a8w8_block", "a8w8_quant": "a8w8_block_quant"}.get(base, base)
                 + ("_packed" if op.endswith("_packed") else ""))
    if base in ("bf16", "gated"):
        return fn(x, w, y=y)
    if base == "fp8_tensor":
        return fn(x, w, s0, y=y)
    if base == "a8w8_block":
        return fn(x, w, s0, s1, y=y)
    return fn(x, w, s1, y=y)


@pytest.mark.parametrize("op", list(skg.OPS))
def test_table_entries_from_graph_replay(op):
    base = op[:-len("_packed")] if op.endswith("_packed") else op
    shapes = _entries(op)
    assert shapes, f"the table has no {op} entries"
    checked = 0
    for (N, K), entries in sorted(shapes.items()):
        Mmax = max(e["rows"] for e in entries)
        p = MAKE[base](Mmax, N, K, seed=0)
        head = base == "fp8_tensor" and N >= 65536
        cols = head_cols(N, 0) if head else None
        if base == "bf16":
            ref = oracle.linear_bf16(p.x, p.w, cols=cols)
        elif base == "gated":
            ref = oracle.linear_gated(p.x, p.w, cols=cols)
        elif base == "fp8_tensor":
            ref = oracle.linear_fp8_tensor(p.x, p.w, p.s0, cols=cols)
        elif base == "a8w8_block":
            ref = oracle.linear_a8w8_block(p.x, p.s0, p.w, p.s1, cols=cols)
        else:
            ref = oracle.linear_a8w8_quant(p.x, p.w, p.s1, cols=cols)[0]
        xd = dev_fp8(p.x) if base == "a8w8_block" else dev_bf16(p.x)
        wd = dev_bf16(p.w) if base in ("bf16", "gated") else dev_fp8(p.w)
        if op.endswith("_packed"):
            wd = skg.skinny_gemm_pack_weight(base, wd)
        s0 = dev_f32(p.s0) if p.s0 is not None else None
        s1 = dev_f32(p.s1) if p.s1 is not None else None
        for e in sorted(entries, key=lambda e: e["rows"]):
            M = e["rows"]
            choice, src = skg.skinny_gemm_query(op, M, N, K)
            assert (choice, src) == (e["choice"], "table"), (op, M, N, K, choice, src, e["choice"])
            s0m = s0[:M] if base == "a8w8_block" else (None if base == "a8w8_quant" else s0)
            y = torch.full((M, N), 3.0, dtype=torch.bfloat16, device="cuda")
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                _call(op, xd[:M], wd, s0m, s1, y)
            g.replay()
            torch.cuda.synchronize()
            bits = host_bits(y)
            if head:
                bits = bits[:, cols]
            say(f"table {op} rows={M} N={N} K={K} {choice}: graph replay")
            assert_parity(bits, ref[:M], f"table {op} rows={M} N={N} K={K} {choice}")
            del g
            checked += 1
        del wd, xd
        torch.cuda.empty_cache()
    assert checked == sum(len(v) for v in shapes.values())

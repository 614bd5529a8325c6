"""Build libskinny_gemm.so for gfx950 in-tree.

    python -m gemv_skinny_gemm_02_amd.build [--jobs N]

Each HIP source is compiled by hipcc for gfx950 only, in parallel, then linked
into gemv_skinny_gemm_02_amd/libskinny_gemm.so beside this file.  Objects go
to _build/ at the repository root.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
import time
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libskinny_gemm.so")
ARCH = "gfx950"

HIP_SOURCES = ["abi.hip", "pack.hip", "calib.hip", "ops_bf16.hip", "ops_gated.hip", "ops_fp8t.hip", "ops_a8w8.hip", "ops_a8w8q.hip",
               "ops_bf16p.hip", "ops_gatedp.hip", "ops_fp8tp.hip", "ops_a8w8p.hip", "ops_a8w8qp.hip", "ops_mt.hip", "ops_pg.hip"]
CXX_SOURCES = ["table.cpp"]

# Packed fp32 VALU ops are kept out of the device code: hipcc -O3 would form
# them from ordinary float code, and this library does not rely on them.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument", "-I", INCLUDE, "-I", CSRC]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def _run(cmd):
    t = time.time()
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines()
                    if "is not a recognized feature for this target" not in l)
    return p.returncode, out, time.time() - t


def build(jobs: int | None = None, verbose: bool = False) -> str:
    """Compile every source and link the library; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    cxx = shutil.which("g++") or "g++"
    jobs = jobs or max(1, min(16, os.cpu_count() or 1))
    cmds = []
    objs = []
    for s in HIP_SOURCES:
        o = os.path.join(BUILD, os.path.splitext(s)[0] + ".o")
        cmds.append([hipcc, *HIP_FLAGS, "-c", os.path.join(CSRC, s), "-o", o])
        objs.append(o)
    for s in CXX_SOURCES:
        o = os.path.join(BUILD, os.path.splitext(s)[0] + ".host.o")
        cmds.append([cxx, *CXX_FLAGS, "-c", os.path.join(CSRC, s), "-o", o])
        objs.append(o)
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_run, cmds))
    failed = False
    for cmd, (rc, out, dt) in zip(cmds, results):
        if verbose or rc:
            print(f"[{dt:5.1f}s] {os.path.basename(cmd[-3])}: rc={rc}", file=sys.stderr)
            if out.strip():
                print(out, file=sys.stderr)
        failed |= rc != 0
    if failed:
        raise RuntimeError("compilation failed")
    tmp = LIB + ".tmp"
    rc, out, _ = _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    if rc:
        print(out, file=sys.stderr)
        raise RuntimeError("link failed")
    os.replace(tmp, LIB)
    return LIB


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args()
    t = time.time()
    print(build(a.jobs, a.verbose), f"({time.time() - t:.1f}s)")


if __name__ == "__main__":
    main()

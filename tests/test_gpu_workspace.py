"""The split-K workspace on the GPU: a call reports and gets the workspace its
dispatch choice needs; without one it is refused before any launch; which
kernel runs does not depend on graph capture (the first call of a process,
captured, gives the eager bits); two streams with their own workspaces run
concurrently and both match the oracle; a graph keeps the workspace it was
captured with after the stream's registration changes."""
import os
import subprocess
import sys
import textwrap

import numpy as np
import pytest
import torch

import gemv_skinny_gemm_02_amd as skg
import synth
from gpu_util import _WS, assert_parity, ensure_workspace, host_bits, reference, run, run_packed, say, to_device, to_device_packed

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    skg.load()
    ensure_workspace()


def _split_variant(op, M):
    """A variant of op that splits K across workgroups and runs M rows."""
    names = skg.variants(op)
    for i, n in enumerate(names):
        if n.startswith("tlds_") and "_s1_" not in n and skg.skinny_gemm_variant_supports(op, i, M):
            return n
    raise AssertionError(f"no split-K variant of {op} at M={M}")


def test_workspace_bytes_match_the_dispatch_choice():
    """skinny_gemm_workspace_bytes equals what the chosen variant needs:
    256 KiB of counters plus S*G*M*N*4 bytes of partials, or 0."""
    seen_split = False
    for op in ("bf16", "bf16_packed", "gated", "a8w8_block", "a8w8_quant_packed"):
        for (M, N, K) in [(1, 4096, 4096), (64, 4096, 4096), (96, 4096, 4096), (128, 6144, 4096),
                          (64, 2048, 2048), (512, 8192, 4096), (300, 1024, 1024)]:
            name, _ = skg.skinny_gemm_query(op, M, N, K)
            need = skg.skinny_gemm_workspace_bytes(op, M, N, K)
            assert need == skg.skinny_gemm_variant_workspace_bytes(op, name, M, N), (op, M, N, K, name)
            parts = name.split("_")
            S = next((int(p[1:]) for p in parts if p.startswith("s") and p[1:].isdigit()), 1)
            G = 2 if op.startswith("gated") else 1
            want = 0 if (S == 1 or name.startswith(("gemv_", "tile_"))) else (256 << 10) + S * G * M * N * 4
            assert need == want, (op, M, N, K, name, need, want)
            seen_split |= need > 0
    assert seen_split


def test_split_k_call_without_workspace_is_refused():
    """With no workspace for its stream, a split-K call returns EUNSUPPORTED and
    leaves y untouched; a workspace one byte short is refused too; the exact
    size runs and matches the oracle."""
    M, N, K = 64, 1024, 2048
    v = _split_variant("bf16", M)
    need = skg.skinny_gemm_variant_workspace_bytes("bf16", v, M, N)
    assert need > 256 << 10
    p = synth.make_bf16(M, N, K, seed=11)
    dev = to_device(p)
    s = torch.cuda.Stream()
    skg.skinny_gemm_set_device_workspace(None)
    try:
        with torch.cuda.stream(s):
            y = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")
            with pytest.raises(skg.SkinnyGemmError) as ei:
                run(p, dev, variant=v, y=y)
            assert ei.value.status == 2 and "workspace" in str(ei.value)
            s.synchronize()
            assert torch.all(y == 7.0)
            short = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
            skg.skinny_gemm_set_workspace(short, stream=s)
            with pytest.raises(skg.SkinnyGemmError):
                run(p, dev, variant=v, y=y)
            skg.skinny_gemm_set_workspace(need, stream=s)
            run(p, dev, variant=v, y=y)
            s.synchronize()
            assert_parity(host_bits(y), reference(p), f"{v} with an exact workspace")
            skg.skinny_gemm_set_workspace(None, stream=s)
    finally:
        skg.skinny_gemm_set_device_workspace(_WS[0])


def test_registration_refusals():
    lib = skg.load()
    s = torch.cuda.current_stream().cuda_stream
    buf = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    assert lib.skinny_gemm_set_workspace(s, buf.data_ptr(), 1000) == 1                 # under 256 KiB
    assert lib.skinny_gemm_set_workspace(s, buf.data_ptr() + 16, 512 << 10) == 2       # alignment
    assert lib.skinny_gemm_set_workspace(s, buf.data_ptr(), 4 << 20) == 1             # past the allocation
    host = np.zeros(2 << 20, dtype=np.uint8)
    hp = (host.ctypes.data + 255) // 256 * 256                                         # aligned host address
    assert lib.skinny_gemm_set_workspace(s, hp, 512 << 10) == 1                       # host memory
    g = torch.cuda.CUDAGraph()
    st = []
    with torch.cuda.graph(g):
        cs = torch.cuda.current_stream().cuda_stream
        st.append(lib.skinny_gemm_set_workspace(cs, buf.data_ptr(), 512 << 10))        # under capture
        buf[:16].fill_(1)
    assert st == [1]
    assert lib.skinny_gemm_set_workspace(s, None, 0) == 0                             # removal is fine


def test_two_streams_with_their_own_workspaces():
    """Split-K calls on two streams, each with its own workspace, interleaved
    with no synchronisation between the streams: both match the oracle and
    give the bits of a serial run."""
    cases = [(synth.make_bf16(64, 4096, 4096, seed=12), "bf16"), (synth.make_bf16(128, 2048, 1024, seed=13), "bf16")]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    want = []
    for (p, op), s in zip(cases, streams):
        v = _split_variant(op, p.M)
        skg.skinny_gemm_set_workspace(skg.skinny_gemm_variant_workspace_bytes(op, v, p.M, p.N), stream=s)
        dev = to_device(p)
        y = torch.empty((p.M, p.N), dtype=torch.bfloat16, device="cuda")
        torch.cuda.synchronize()
        want.append((p, dev, v, y, s, reference(p)))
    serial = []
    for p, dev, v, y, s, ref in want:
        serial.append(host_bits(run(p, dev, variant=v)))
    torch.cuda.synchronize()
    for _ in range(20):
        for p, dev, v, y, s, ref in want:
            with torch.cuda.stream(s):
                run(p, dev, variant=v, y=y)
    torch.cuda.synchronize()
    for (p, dev, v, y, s, ref), bits in zip(want, serial):
        got = host_bits(y)
        assert_parity(got, ref, f"{v} M={p.M} N={p.N} on its own stream")
        assert np.array_equal(got, bits)
    for s in streams:
        skg.skinny_gemm_set_workspace(None, stream=s)


def test_graph_keeps_its_workspace_after_reregistration():
    """A graph captured on a stream keeps the workspace it was captured with:
    after the stream gets a larger workspace and an eager call uses it, the
    graph still replays the first bits."""
    M, N, K = 64, 4096, 2048
    v = _split_variant("bf16", M)
    p = synth.make_bf16(M, N, K, seed=14)
    dev = to_device(p)
    s = torch.cuda.Stream()
    skg.skinny_gemm_set_workspace(skg.skinny_gemm_variant_workspace_bytes("bf16", v, M, N), stream=s)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    with torch.cuda.stream(s):
        run(p, dev, variant=v, y=y)
    s.synchronize()
    first = host_bits(y)
    assert_parity(first, reference(p), v)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        run(p, dev, variant=v, y=y)
    # a bigger problem needs a bigger workspace: register it and run eagerly
    p2 = synth.make_bf16(128, N, K, seed=15)
    dev2 = to_device(p2)
    skg.skinny_gemm_set_workspace(skg.skinny_gemm_variant_workspace_bytes("bf16", v, 128, N) + (1 << 20), stream=s)
    with torch.cuda.stream(s):
        y2 = run(p2, dev2, variant=v)
    s.synchronize()
    assert_parity(host_bits(y2), reference(p2), f"{v} M=128 eager")
    for _ in range(3):
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(y), first), "replay after re-registration"
    skg.skinny_gemm_set_workspace(None, stream=s)


def test_first_call_captured_in_a_fresh_process(tmp_path):
    """In a fresh process whose first GEMM call is captured into a graph, the
    replayed bits equal an eager call's, for a workload key whose dispatch
    choice splits K."""
    key = None
    for (N, K) in synth.SWEEP_NK:
        for M in synth.SWEEP_M:
            if skg.skinny_gemm_workspace_bytes("bf16_packed", M, N, K) > 0:
                key = (M, N, K)
                break
        if key:
            break
    assert key, "no workload key splits K"
    M, N, K = key
    out = tmp_path / "y.npy"
    script = textwrap.dedent(f"""
        import sys
        sys.path.insert(0, {ROOT!r})
        import numpy as np, torch
        import gemv_skinny_gemm_02_amd as skg, synth
        torch.cuda.set_device(0)
        p = synth.make_bf16({M}, {N}, {K}, seed=16)
        x = torch.from_numpy(p.x.view(np.int16)).view(torch.bfloat16).cuda()
        w = torch.from_numpy(p.w.view(np.int16)).view(torch.bfloat16).cuda()
        skg.skinny_gemm_set_device_workspace(64 << 20)
        wp = skg.skinny_gemm_pack_weight("bf16", w)
        y = torch.empty(({M}, {N}), dtype=torch.bfloat16, device="cuda")
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            skg.skinny_gemm_bf16_packed(x, wp, y=y)     # the process's first GEMM call
        g.replay(); g.replay()
        torch.cuda.synchronize()
        graph_bits = y.cpu().view(torch.int16).numpy().copy()
        eager = skg.skinny_gemm_bf16_packed(x, wp)
        torch.cuda.synchronize()
        same = np.array_equal(graph_bits, eager.cpu().view(torch.int16).numpy())
        np.save({str(out)!r}, graph_bits.view(np.uint16))
        print("CHOICE", skg.skinny_gemm_query("bf16_packed", {M}, {N}, {K}))
        print("SAME" if same else "DIFFERENT", flush=True)
    """)
    say(f"fresh process, first call captured: bf16_packed M={M} N={N} K={K}")
    r = subprocess.run([sys.executable, "-c", script], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "SAME" in r.stdout, r.stdout
    p = synth.make_bf16(M, N, K, seed=16)
    assert_parity(np.load(out), reference(p), f"captured first call M={M} N={N} K={K}")


def test_split_slices_without_waits(tmp_path):
    """Tiles that split K four or eight ways add each slice of a tile in the
    split that owns it, after a bounded wait for the tile's other splits.
    With the waits switched off ($SKINNY_GEMM_SPLIT_WAIT=0, read once per
    process, so in a fresh one) the last split to arrive adds every slice
    itself.  Both ways give the same bits, for every such variant of the
    packed bf16 and gated forms, on N divisible by 4 (16-byte partial rows)
    and not, and they pass the oracle."""
    M = 64
    shapes = [("bf16", 1024, 4096), ("bf16", 1030, 2048), ("gated", 512, 4096)]
    cases = []
    for kind, N, K in shapes:
        op = kind + "_packed"
        for i, n in enumerate(skg.variants(op)):
            if n.startswith("tlds_") and ("_s4_" in n or "_s8_" in n) and skg.skinny_gemm_variant_supports(op, i, M):
                cases.append((kind, N, K, n))
    assert len(cases) >= 6
    out = tmp_path / "nowait.npz"
    script = textwrap.dedent(f"""
        import sys
        sys.path.insert(0, {ROOT!r}); sys.path.insert(0, {os.path.join(ROOT, 'tests')!r})
        import numpy as np, torch
        import gemv_skinny_gemm_02_amd as skg, synth
        from gpu_util import to_device_packed, run_packed, host_bits
        torch.cuda.set_device(0)
        skg.skinny_gemm_set_device_workspace(64 << 20)
        res = {{}}
        for i, (kind, N, K, v) in enumerate({cases!r}):
            p = getattr(synth, "make_" + kind)({M}, N, K, seed=21)
            y = run_packed(p, to_device_packed(p), variant=v)
            torch.cuda.synchronize()
            res["c%d" % i] = host_bits(y)
        np.savez({str(out)!r}, **res)
        print("DONE", flush=True)
    """)
    say(f"split slices without waits: {len(cases)} cases in a fresh process")
    env = dict(os.environ, SKINNY_GEMM_SPLIT_WAIT="0")
    r = subprocess.run([sys.executable, "-c", script], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "DONE" in r.stdout, r.stdout
    nowait = np.load(out)
    for i, (kind, N, K, v) in enumerate(cases):
        p = getattr(synth, "make_" + kind)(M, N, K, seed=21)
        y = host_bits(run_packed(p, to_device_packed(p), variant=v))
        assert np.array_equal(y, nowait[f"c{i}"]), f"{kind} N={N} K={K} {v}: waits on/off differ"
        assert_parity(y, reference(p), f"{kind} N={N} K={K} {v}")

"""The C ABI on the GPU: status codes, edge cases, guard bytes, and the
determinism of results and of dispatch."""
import ctypes

import numpy as np
import pytest
import torch

import gemv_skinny_gemm_02_amd as skg
import oracle
import synth
from gpu_util import ensure_workspace, assert_parity, dev_bf16, dev_f32, dev_fp8, host_bits, reference, run, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    skg.load()
    ensure_workspace()


def _raw(fn, *args):
    lib = skg.load()
    st = getattr(lib, fn)(*args)
    return st, lib.skinny_gemm_last_error().decode()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def test_empty_is_noop():
    x = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((8, 64), dtype=torch.bfloat16, device="cuda")
    y = torch.full((4, 8), 7.0, dtype=torch.bfloat16, device="cuda")
    for M, N in ((0, 8), (4, 0)):
        st, _ = _raw("skinny_gemm_bf16", x.data_ptr(), w.data_ptr(), None, y.data_ptr(), M, N, 64, _stream())
        assert st == 0
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)
    e = skg.skinny_gemm_bf16(torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda"), w)
    assert e.shape == (0, 8)


def test_k_zero_writes_zeros():
    for kind in ("bf16", "gated", "fp8_tensor", "a8w8_block"):
        p = {"bf16": synth.make_bf16, "gated": synth.make_gated, "fp8_tensor": synth.make_fp8_tensor,
             "a8w8_block": synth.make_a8w8_block}[kind](3, 40, 16)
        x, w, s0, s1 = to_device(p)
        y = torch.full((3, 40), 5.0, dtype=torch.bfloat16, device="cuda")
        lib = skg.load()
        if kind == "a8w8_block":
            st = lib.skinny_gemm_a8w8_block(x.data_ptr(), w.data_ptr(), s0.data_ptr(), s1.data_ptr(), y.data_ptr(),
                                            3, 40, 0, _stream())
        else:
            st = getattr(lib, "skinny_gemm_" + kind)(x.data_ptr(), w.data_ptr(), s0.data_ptr() if s0 is not None else None,
                                                     y.data_ptr(), 3, 40, 0, _stream())
        assert st == 0, lib.skinny_gemm_last_error()
        torch.cuda.synchronize()
        assert torch.all(y == 0), kind


def test_status_codes():
    x = torch.zeros((2, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((16, 64), dtype=torch.bfloat16, device="cuda")
    y = torch.zeros((2, 16), dtype=torch.bfloat16, device="cuda")
    s = _stream()
    assert _raw("skinny_gemm_bf16", x.data_ptr(), w.data_ptr(), None, y.data_ptr(), -1, 16, 64, s)[0] == 1
    assert _raw("skinny_gemm_bf16", None, w.data_ptr(), None, y.data_ptr(), 2, 16, 64, s)[0] == 1
    st, msg = _raw("skinny_gemm_bf16", x.data_ptr(), w.data_ptr(), None, y.data_ptr(), 2, 16, 60, s)
    assert st == 2 and "K" in msg
    st, msg = _raw("skinny_gemm_bf16", x.data_ptr() + 2, w.data_ptr(), None, y.data_ptr(), 2, 16, 56, s)
    assert st == 2 and "aligned" in msg
    # y overlapping x
    st, msg = _raw("skinny_gemm_bf16", x.data_ptr(), w.data_ptr(), None, x.data_ptr(), 2, 16, 64, s)
    assert st == 1 and "overlap" in msg
    # host memory is refused on the host, before any launch
    host = np.zeros((2, 64), np.uint16)
    st, msg = _raw("skinny_gemm_bf16", host.ctypes.data, w.data_ptr(), None, y.data_ptr(), 2, 16, 64, s)
    assert st == 1 and "device memory" in msg
    # fp8 needs K % 16
    w8 = torch.zeros((16, 64), dtype=torch.uint8, device="cuda")
    sc = torch.ones(1, dtype=torch.float32, device="cuda")
    st, _ = _raw("skinny_gemm_fp8_tensor", x.data_ptr(), w8.data_ptr(), sc.data_ptr(), y.data_ptr(), 2, 16, 56, s)
    assert st == 2
    # fp8 tensor without its scale
    st, _ = _raw("skinny_gemm_fp8_tensor", x.data_ptr(), w8.data_ptr(), None, y.data_ptr(), 2, 16, 64, s)
    assert st == 1
    # knobs are reserved
    st, _ = _raw("skinny_gemm_run_variant", 0, 0, ctypes.byref(ctypes.c_int(1)), x.data_ptr(), w.data_ptr(), None,
                 None, y.data_ptr(), 2, 16, 64, s)
    assert st == 1
    # a variant that is not compiled for the rows bucket
    names = skg.variants("gated")
    st, _ = _raw("skinny_gemm_run_variant", 1, names.index("gemv_r4_k4_p1"), None, x.data_ptr(), w.data_ptr(),
                 None, None, y.data_ptr(), 2, 8, 64, s)
    assert st == 0
    xw = torch.zeros((16, 64), dtype=torch.bfloat16, device="cuda")
    yw = torch.zeros((16, 8), dtype=torch.bfloat16, device="cuda")
    st, _ = _raw("skinny_gemm_run_variant", 1, names.index("gemv_r4_k4_p1"), None, xw.data_ptr(), w.data_ptr(),
                 None, None, yw.data_ptr(), 16, 8, 64, s)
    assert st == 2


def test_quant_status_codes_and_scale_guards():
    """The entry point that quantises x: its x-scale output is refused when it
    overlaps an operand, and the call when its w scales are missing; K = 0
    writes zeros and no scale; the scales it writes stay inside their
    [M, ceil(K/128)] buffer."""
    M, N, K = 17, 77, 272                                   # 3 groups, the last of 16
    p = synth.make_a8w8_quant(M, N, K, seed=4)
    x, w, _, ws = to_device(p)
    y = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    kb = 3
    s = _stream()
    buf = torch.full((M * kb + 1024,), -7.0, dtype=torch.float32, device="cuda")
    xs = buf[:M * kb]
    fn = "skinny_gemm_a8w8_block_quant"
    st, msg = _raw(fn, x.data_ptr(), w.data_ptr(), ws.data_ptr(), y.data_ptr(), y.data_ptr(), M, N, K, s)
    assert st == 1 and "overlap" in msg, msg
    st, msg = _raw(fn, x.data_ptr(), w.data_ptr(), ws.data_ptr(), x.data_ptr(), y.data_ptr(), M, N, K, s)
    assert st == 1 and "overlap" in msg, msg
    st, msg = _raw(fn, x.data_ptr(), w.data_ptr(), None, xs.data_ptr(), y.data_ptr(), M, N, K, s)
    assert st == 1, msg
    # K = 0: y = 0 and nothing written to the scales
    y.fill_(5.0)
    st, msg = _raw(fn, x.data_ptr(), w.data_ptr(), ws.data_ptr(), xs.data_ptr(), y.data_ptr(), M, N, 0, s)
    assert st == 0, msg
    torch.cuda.synchronize()
    assert torch.all(y == 0) and torch.all(buf == -7.0)
    # a real call: scales exact, nothing written past them, y at the parity bar
    yb = torch.full((M * N + 4096,), 12345, dtype=torch.int16, device="cuda")
    y2 = yb[:M * N].view(torch.bfloat16).view(M, N)
    skg.skinny_gemm_a8w8_block_quant(x, w, ws, x_scales=xs.view(M, kb), y=y2)
    torch.cuda.synchronize()
    assert torch.all(buf[M * kb:] == -7.0) and torch.all(yb[M * N:] == 12345)
    ref, _, want = oracle.linear_a8w8_quant(p.x, p.w, p.s1)
    assert np.array_equal(xs.cpu().numpy().reshape(M, kb).view(np.uint32), want.view(np.uint32))
    assert_parity(host_bits(y2), ref, "a8w8_quant guards")


def test_short_allocation_refused():
    """A W that is shorter than N*K*2 bytes is refused on the host."""
    hip = ctypes.CDLL("libamdhip64.so")
    w = torch.empty((4 << 20) // 2, dtype=torch.bfloat16, device="cuda")    # 4 MiB
    base, size = ctypes.c_void_p(), ctypes.c_size_t()
    assert hip.hipMemGetAddressRange(ctypes.byref(base), ctypes.byref(size), ctypes.c_void_p(w.data_ptr())) == 0
    N, K = 1 << 20, 4096                                  # claims 8 GiB
    need = N * K * 2
    if base.value + size.value >= w.data_ptr() + need:
        pytest.skip("allocator segment is unexpectedly large")
    x = torch.zeros((1, K), dtype=torch.bfloat16, device="cuda")
    y = torch.zeros((1, N), dtype=torch.bfloat16, device="cuda")
    st, msg = _raw("skinny_gemm_bf16", x.data_ptr(), w.data_ptr(), None, y.data_ptr(), 1, N, K, _stream())
    assert st == 1 and "W needs" in msg, msg


def test_guard_bytes_untouched():
    """Writes stay inside y: a guard region after y keeps its bytes."""
    for kind, M, N, K in (("bf16", 3, 77, 264), ("gated", 20, 50, 264), ("fp8_tensor", 2, 77, 272),
                          ("a8w8_block", 17, 77, 272)):
        p = {"bf16": synth.make_bf16, "gated": synth.make_gated, "fp8_tensor": synth.make_fp8_tensor,
             "a8w8_block": synth.make_a8w8_block}[kind](M, N, K, seed=3)
        dev = to_device(p)
        buf = torch.full((M * N + 4096,), 12345, dtype=torch.int16, device="cuda")
        y = buf[:M * N].view(torch.bfloat16).view(M, N)
        run(p, dev, y=y)
        torch.cuda.synchronize()
        assert torch.all(buf[M * N:] == 12345), kind
        assert_parity(host_bits(y), reference(p), kind)


def test_repeat_bit_identical_and_graph_replay():
    """10 repeats are bit-identical; a captured graph replays the same bits,
    with eager work and synchronisation between replays."""
    cases = [synth.make_bf16(8, 4096, 4096), synth.make_gated(6, 1024, 4096),
             synth.make_fp8_tensor(2, 4096, 4096), synth.make_a8w8_block(32, 8192, 4096),
             synth.make_bf16(128, 4096, 4096)]
    for p in cases:
        say(f"determinism {p.kind} M={p.M} N={p.N} K={p.K}")
        dev = to_device(p)
        first = host_bits(run(p, dev))
        for _ in range(9):
            assert np.array_equal(host_bits(run(p, dev)), first)
        y = torch.empty((p.M, p.N), dtype=torch.bfloat16, device="cuda")
        run(p, dev, y=y)                      # warm-up outside capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run(p, dev, y=y)
        for _ in range(3):
            y.zero_()
            junk = torch.randn(1 << 16, device="cuda") * 2   # eager work between replays
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert np.array_equal(host_bits(y), first), f"graph replay {p.kind}"
            del junk


def test_dispatch_deterministic():
    a = [skg.skinny_gemm_query(k, M, N, K) for k in skg.OPS for M in (1, 5, 16, 100, 300)
         for (N, K) in ((4096, 4096), (1024, 1024))]
    b = [skg.skinny_gemm_query(k, M, N, K) for k in skg.OPS for M in (1, 5, 16, 100, 300)
         for (N, K) in ((4096, 4096), (1024, 1024))]
    assert a == b


def test_split_k_counters_and_graph_replay():
    """Split-K variants combine partials through per-tile arrival counters that
    each launch leaves at zero: repeated calls, calls on other shapes in
    between, and graph replays all give the eager bits."""
    names = skg.variants("bf16")
    split = [n for n in names if n.startswith("tlds_") and "_s1_" not in n]
    assert split
    cases = [(64, 4096, 4096), (24, 1000, 2064), (128, 2048, 1024), (17, 4096, 512)]
    first = {}
    for (M, N, K) in cases:
        p = synth.make_bf16(M, N, K, seed=5)
        dev = to_device(p)
        ref = reference(p)
        for v in split:
            if not skg.skinny_gemm_variant_supports("bf16", names.index(v), M):
                continue
            y = run(p, dev, variant=v)
            torch.cuda.synchronize()
            bits = host_bits(y)
            assert_parity(bits, ref, f"{v} M={M} N={N} K={K}")
            first[(M, N, K, v)] = (p, dev, bits)
    # interleave shapes and variants, then repeat: same bits every time
    for _ in range(2):
        for (M, N, K, v), (p, dev, bits) in first.items():
            assert np.array_equal(host_bits(run(p, dev, variant=v)), bits), (M, N, K, v)
    # graph replay of a split-K variant, eager work in between
    (M, N, K, v), (p, dev, bits) = next(iter(first.items()))
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    run(p, dev, variant=v, y=y)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(3):
            run(p, dev, variant=v, y=y)
    for _ in range(3):
        y.zero_()
        junk = torch.randn(1 << 16, device="cuda") * 2
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(y), bits), f"graph replay {v}"
        del junk


def test_calib_kernels_statuses():
    """The measurement kernels run, and refuse what the header says they refuse."""
    buf = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    s = _stream()
    say("calib read 1 MiB, grid 64")
    assert _raw("skinny_gemm_calib_read", buf.data_ptr(), buf.numel(), 64, 0, sink.data_ptr(), s)[0] == 0
    skg.skinny_gemm_calib_read(buf, 2048, sink)
    skg.skinny_gemm_calib_read(buf, 300, sink, sweep=True)
    flops = skg.skinny_gemm_calib_mfma(8, 16, sink)
    assert flops == 8 * 16 * 4 * 8 * 32768
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0            # zero data never folds to the sink pattern
    host = np.zeros(1024, dtype=np.uint8)
    st, msg = _raw("skinny_gemm_calib_read", host.ctypes.data, 1024, 4, 0, sink.data_ptr(), s)
    assert st == 1 and "device memory" in msg
    assert _raw("skinny_gemm_calib_read", buf.data_ptr() + 8, 1024, 4, 0, sink.data_ptr(), s)[0] == 2
    assert _raw("skinny_gemm_calib_read", buf.data_ptr(), 1000, 4, 0, sink.data_ptr(), s)[0] == 2
    assert _raw("skinny_gemm_calib_read", buf.data_ptr(), 8 << 30, 4, 0, sink.data_ptr(), s)[0] == 1   # past the allocation
    assert _raw("skinny_gemm_calib_read", buf.data_ptr(), 1024, 0, 0, sink.data_ptr(), s)[0] == 1
    assert _raw("skinny_gemm_calib_read", buf.data_ptr(), 1024, 4, 2, sink.data_ptr(), s)[0] == 1
    hsink = np.zeros(256, dtype=np.int32)
    assert _raw("skinny_gemm_calib_read", buf.data_ptr(), 1024, 4, 0, hsink.ctypes.data, s)[0] == 1
    assert _raw("skinny_gemm_calib_mfma", 0, 16, sink.data_ptr(), s)[0] == 1
    assert _raw("skinny_gemm_calib_mfma", 8, 0, sink.data_ptr(), s)[0] == 1
    assert _raw("skinny_gemm_calib_mfma", 8, 16, hsink.ctypes.data, s)[0] == 1
    torch.cuda.synchronize()

"""Mid-M rows (144 .. 512: speculative verification and drafting) and small-N
weights on the GPU: every tile variant of the bf16 form, row-major and packed,
on a ragged small shape element by element; table dispatch at the full sweep
shapes and at the small-N shapes on every output; all against the CPU
oracle."""
import numpy as np
import pytest
import torch

import gemv_skinny_gemm_02_amd as skg
import oracle
import synth
from gpu_util import (ensure_workspace, assert_parity, dev_bf16, dev_f32, dev_fp8, host_bits, reference, run, run_packed, say, to_device,
                      to_device_packed)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    skg.load()
    ensure_workspace()


@pytest.mark.parametrize("op", ["bf16", "bf16_packed"])
def test_every_variant_mid_m(op):
    """M = 300 spans three launch rows of 128 with a ragged last one; N and K
    are ragged against every tile."""
    N, K = 257, 1032
    names = skg.variants(op)
    for M in (129, 300):
        p = synth.make_bf16(M, N, K, seed=5)
        dev = to_device_packed(p) if op.endswith("_packed") else to_device(p)
        ref = reference(p)
        ran = 0
        for i, name in enumerate(names):
            if not skg.skinny_gemm_variant_supports(op, i, M):
                continue
            say(f"{op} M={M} N={N} K={K} variant={name}")
            y = run_packed(p, dev, variant=name) if op.endswith("_packed") else run(p, dev, variant=name)
            torch.cuda.synchronize()
            assert_parity(host_bits(y), ref, f"{op} {name} M={M}")
            ran += 1
        assert ran > 0


def test_mid_m_full_shapes():
    """Table dispatch at every mid-M workload row on the five sweep shapes, both
    layouts, every output (the oracle at the largest M, sliced: row m depends
    on row m of x only)."""
    for (N, K) in synth.SWEEP_NK:
        base = synth.make_bf16(max(synth.MID_M), N, K, seed=0)
        w = dev_bf16(base.w)
        wp = skg.skinny_gemm_pack_weight("bf16", w)
        full = oracle.linear_bf16(base.x, base.w)
        for M in synth.MID_M:
            x = dev_bf16(base.x[:M])
            ref = full[:M]
            say(f"bf16 mid M={M} N={N} K={K} -> {skg.skinny_gemm_query('bf16', M, N, K)}, "
                f"packed -> {skg.skinny_gemm_query('bf16_packed', M, N, K)}")
            y = skg.skinny_gemm_bf16(x, w)
            yp = skg.skinny_gemm_bf16_packed(x, wp)
            torch.cuda.synchronize()
            assert_parity(host_bits(y), ref, f"bf16 M={M} N={N} K={K}")
            assert_parity(host_bits(yp), ref, f"bf16_packed M={M} N={N} K={K}")


def test_small_n_full_shapes():
    """Small-N bf16 weights (N = 64 .. 2048, K = 4096), table dispatch, both
    layouts, every output against the oracle; and two calls in a row give the
    same bits (the cross-workgroup K split adds its partials in a fixed
    order)."""
    for (N, K) in synth.SMALLN_NK:
        base = synth.make_bf16(max(synth.SMALLN_M), N, K, seed=0)
        w = dev_bf16(base.w)
        wp = skg.skinny_gemm_pack_weight("bf16", w)
        for M in synth.SMALLN_M:
            x = dev_bf16(base.x[:M])
            ref = oracle.linear_bf16(base.x[:M], base.w)
            say(f"bf16 small-N M={M} N={N} K={K} -> {skg.skinny_gemm_query('bf16', M, N, K)}, "
                f"packed -> {skg.skinny_gemm_query('bf16_packed', M, N, K)}")
            y, y2 = skg.skinny_gemm_bf16(x, w), skg.skinny_gemm_bf16(x, w)
            yp, yp2 = skg.skinny_gemm_bf16_packed(x, wp), skg.skinny_gemm_bf16_packed(x, wp)
            torch.cuda.synchronize()
            assert_parity(host_bits(y), ref, f"bf16 M={M} N={N} K={K}")
            assert_parity(host_bits(yp), ref, f"bf16_packed M={M} N={N} K={K}")
            assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
            assert torch.equal(yp.view(torch.int16), yp2.view(torch.int16))


@pytest.mark.parametrize("op", ["a8w8_block", "a8w8_block_packed"])
def test_every_a8w8_variant_mid_m(op):
    """A8W8 block scale at mid-M rows (the verify and drafter rows of the A8W8
    tables), every variant, ragged N and K, element by element."""
    N, K = 257, 1040
    names = skg.variants(op)
    for M in (129, 300):
        p = synth.make_a8w8_block(M, N, K, seed=6)
        dev = to_device_packed(p) if op.endswith("_packed") else to_device(p)
        ref = reference(p)
        ran = 0
        for i, name in enumerate(names):
            if not skg.skinny_gemm_variant_supports(op, i, M):
                continue
            say(f"{op} M={M} N={N} K={K} variant={name}")
            y = run_packed(p, dev, variant=name) if op.endswith("_packed") else run(p, dev, variant=name)
            torch.cuda.synchronize()
            assert_parity(host_bits(y), ref, f"{op} {name} M={M}")
            ran += 1
        assert ran > 0


def test_a8w8_mid_m_full_shapes():
    """Table dispatch of A8W8 at every mid-M workload row on (32768, 1024) and
    (8192, 4096), both layouts, every output."""
    for (N, K) in synth.A8W8_NK:
        base = synth.make_a8w8_block(max(synth.MID_M), N, K, seed=0)
        w, ws = dev_fp8(base.w), dev_f32(base.s1)
        wp = skg.skinny_gemm_pack_weight("a8w8_block", w)
        full = oracle.linear_a8w8_block(base.x, base.s0, base.w, base.s1)
        for M in synth.MID_M:
            x, xs = dev_fp8(base.x[:M]), dev_f32(base.s0[:M])
            ref = full[:M]
            say(f"a8w8 mid M={M} N={N} K={K} -> {skg.skinny_gemm_query('a8w8_block', M, N, K)}, "
                f"packed -> {skg.skinny_gemm_query('a8w8_block_packed', M, N, K)}")
            y = skg.skinny_gemm_a8w8_block(x, w, xs, ws)
            yp = skg.skinny_gemm_a8w8_block_packed(x, wp, xs, ws)
            torch.cuda.synchronize()
            assert_parity(host_bits(y), ref, f"a8w8_block M={M} N={N} K={K}")
            assert_parity(host_bits(yp), ref, f"a8w8_block_packed M={M} N={N} K={K}")

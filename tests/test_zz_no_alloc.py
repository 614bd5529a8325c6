"""skinny_gemm_run_static through the C ABI: the entry point for callers that
cannot allocate, with its split-K partials in the library's static device
scratch.  Two calls in a row, the second on a smaller input, each give the
bits of the existing entry point of the same form (the same dispatch choice
runs; the result is checked at the parity bar against the oracle too); a call
that needs more partials than the scratch holds is refused before launch."""

import numpy as np
import pytest
import torch

import gemv_skinny_gemm_02_amd as skg
import oracle
import synth
from gpu_util import assert_parity, dev_bf16, ensure_workspace, host_bits, say

pytestmark = pytest.mark.gpu

KB = 256 << 10          # the counters that precede the partials in a workspace


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    skg.load()
    ensure_workspace()


def _static_c(op, x, w_ptr, y, M, N, K):
    """skinny_gemm_run_static through ctypes, on the current stream."""
    lib = skg.load()
    st = lib.skinny_gemm_run_static(skg.OPS[op], x.data_ptr(), w_ptr, None, None, y.data_ptr(), M, N, K,
                                    torch.cuda.current_stream().cuda_stream)
    return st, lib.skinny_gemm_last_error().decode()


def _split_keys(op):
    """Workload keys (sweep and small-N shapes, decode and mid-M rows) whose
    dispatch choice splits K and fits the scratch, largest input first."""
    cap = skg.skinny_gemm_static_scratch_bytes()
    keys = []
    for (N, K) in tuple(synth.SWEEP_NK) + tuple(synth.SMALLN_NK):
        for M in tuple(synth.SWEEP_M) + tuple(synth.MID_M):
            need = skg.skinny_gemm_workspace_bytes(op, M, N, K)
            if need > 0 and need - KB <= cap:
                keys.append((M, N, K))
    return sorted(keys, key=lambda k: -k[0] * k[1] * k[2])


@pytest.mark.parametrize("op", ["bf16_packed", "bf16"])
def test_static_matches_entry_point_twice_second_smaller(op):
    keys = _split_keys(op)
    assert len(keys) >= 2, f"fewer than two split-K keys of {op}: {keys}"
    big, small = keys[0], keys[-1]
    assert small[0] * small[1] * small[2] < big[0] * big[1] * big[2]
    for (M, N, K) in (big, small):
        p = synth.make_bf16(M, N, K, seed=21)
        x, w = dev_bf16(p.x), dev_bf16(p.w)
        if op == "bf16_packed":
            wp = skg.skinny_gemm_pack_weight("bf16", w)
            w_ptr = wp.data.data_ptr()
            want = skg.skinny_gemm_bf16_packed(x, wp)
        else:
            w_ptr = w.data_ptr()
            want = skg.skinny_gemm_bf16(x, w)
        y = torch.full((M, N), 9.0, dtype=torch.bfloat16, device="cuda")
        say(f"run_static {op} M={M} N={N} K={K} -> {skg.skinny_gemm_query(op, M, N, K)} "
            f"(workspace {skg.skinny_gemm_workspace_bytes(op, M, N, K)} bytes)")
        st, msg = _static_c(op, x, w_ptr, y, M, N, K)
        assert st == 0, msg
        torch.cuda.synchronize()
        got, ref_bits = host_bits(y), host_bits(want)
        assert np.array_equal(got, ref_bits), f"{op} M={M} N={N} K={K}: static differs from the entry point"
        assert_parity(got, oracle.dec_bf16(ref_bits), f"{op} M={M} against the entry point")
        assert_parity(got, oracle.linear_bf16(p.x, p.w), f"{op} M={M} against the oracle")


def test_static_refuses_more_than_the_scratch():
    """A call whose dispatch choice needs more partials than the static
    scratch holds returns EUNSUPPORTED with a message and leaves y alone."""
    cap = skg.skinny_gemm_static_scratch_bytes()
    key = None
    for (M, N, K) in [(512, 8192, 1024), (512, 16384, 1024), (512, 8192, 512)]:
        need = skg.skinny_gemm_workspace_bytes("bf16", M, N, K)
        if need - KB > cap:
            key = (M, N, K)
            break
    assert key, "no key needs more than the static scratch"
    M, N, K = key
    x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((N, K), dtype=torch.bfloat16, device="cuda")
    y = torch.full((M, N), 5.0, dtype=torch.bfloat16, device="cuda")
    st, msg = _static_c("bf16", x, w.data_ptr(), y, M, N, K)
    assert st == 2 and "static scratch" in msg, (st, msg)
    torch.cuda.synchronize()
    assert torch.all(y == 5.0)

"""Helpers shared by the GPU tests: move generator outputs to the device, run
the library, compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import gemv_skinny_gemm_02_amd as skg
import oracle


# Split-K workspace the GPU tests register for the device: enough for every
# table entry they run (the largest, A8W8 32768 x 1024 at M = 512 with S = 4,
# takes 256 MiB of partials).
TEST_WORKSPACE_BYTES = 512 << 20
_WS = []


def ensure_workspace() -> None:
    """Register the tests' device-wide split-K workspace once per process."""
    if not _WS:
        _WS.append(skg.skinny_gemm_set_device_workspace(TEST_WORKSPACE_BYTES))


def say(*a) -> None:
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev_fp8(b: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(b)).view(torch.float8_e4m3fn).cuda()


def dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def host_bits(y: torch.Tensor) -> np.ndarray:
    return y.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def to_device(p):
    """Device tensors (x, W, s0, s1) of a synth.Problem."""
    if p.kind in ("bf16", "gated"):
        return dev_bf16(p.x), dev_bf16(p.w), None, None
    if p.kind == "fp8_tensor":
        return dev_bf16(p.x), dev_fp8(p.w), dev_f32(p.s0), None
    if p.kind == "a8w8_quant":       # s0: the x scales the call writes
        kb = -(-p.K // 128)
        return dev_bf16(p.x), dev_fp8(p.w), torch.full((p.M, kb), -1.0, device="cuda"), dev_f32(p.s1)
    return dev_fp8(p.x), dev_fp8(p.w), dev_f32(p.s0), dev_f32(p.s1)


def run(p, dev=None, variant=None, y=None):
    """Run the library on problem p (dispatch, or one variant)."""
    x, w, s0, s1 = dev if dev is not None else to_device(p)
    if variant is not None:
        return skg.skinny_gemm_run_variant(p.kind, variant, x, w, s0, s1, y=y)
    if p.kind == "bf16":
        return skg.skinny_gemm_bf16(x, w, y=y)
    if p.kind == "gated":
        return skg.skinny_gemm_gated(x, w, y=y)
    if p.kind == "fp8_tensor":
        return skg.skinny_gemm_fp8_tensor(x, w, s0, y=y)
    if p.kind == "a8w8_quant":
        return skg.skinny_gemm_a8w8_block_quant(x, w, s1, x_scales=s0, y=y)
    return skg.skinny_gemm_a8w8_block(x, w, s0, s1, y=y)


def to_device_packed(p):
    """Device tensors (x, W_packed, s0, s1) of a synth.Problem, the weight
    packed by the library for the problem's form."""
    x, w, s0, s1 = to_device(p)
    return x, skg.skinny_gemm_pack_weight(p.kind, w), s0, s1


def run_packed(p, dev=None, variant=None, y=None):
    """Run the packed form of problem p (dispatch, or one variant)."""
    x, wp, s0, s1 = dev if dev is not None else to_device_packed(p)
    if variant is not None:
        return skg.skinny_gemm_run_variant(p.kind + "_packed", variant, x, wp, s0, s1, y=y)
    if p.kind == "bf16":
        return skg.skinny_gemm_bf16_packed(x, wp, y=y)
    if p.kind == "gated":
        return skg.skinny_gemm_gated_packed(x, wp, y=y)
    if p.kind == "fp8_tensor":
        return skg.skinny_gemm_fp8_tensor_packed(x, wp, s0, y=y)
    if p.kind == "a8w8_quant":
        return skg.skinny_gemm_a8w8_block_quant_packed(x, wp, s1, x_scales=s0, y=y)
    return skg.skinny_gemm_a8w8_block_packed(x, wp, s0, s1, y=y)


def reference(p, cols=None) -> np.ndarray:
    if p.kind == "bf16":
        return oracle.linear_bf16(p.x, p.w, cols=cols)
    if p.kind == "gated":
        return oracle.linear_gated(p.x, p.w, cols=cols)
    if p.kind == "fp8_tensor":
        return oracle.linear_fp8_tensor(p.x, p.w, p.s0, cols=cols)
    if p.kind == "a8w8_quant":
        return oracle.linear_a8w8_quant(p.x, p.w, p.s1, cols=cols)[0]
    return oracle.linear_a8w8_block(p.x, p.s0, p.w, p.s1, cols=cols)


def assert_parity(y_bits: np.ndarray, ref: np.ndarray, what: str) -> None:
    r = oracle.parity(y_bits, ref)
    assert r.ok, f"{what}: {r.msg}"

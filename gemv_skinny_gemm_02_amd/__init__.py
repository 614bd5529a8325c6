"""Python binding of libskinny_gemm.so, the MI355X (gfx950) skinny decode-linear
library:  y[M, N] = x[M, K] . W[N, K]^T  for M = 1..128 rows.

The binding only marshals arguments: it checks dtypes, shapes and devices of
torch tensors, passes their device pointers and the current HIP stream to the C
entry points of the same names, and raises on a non-zero status.  Every step of
the computation runs in the library's HIP kernels.  torch supplies device
memory and streams only.

Entry points (see include/skinny_gemm.h for the contract):
    skinny_gemm_bf16(x, W)                   bf16 x [M,K], bf16 W [N,K]
    skinny_gemm_gated(x, W)                  W = [2N,K]: gate rows then up rows
    skinny_gemm_fp8_tensor(x, W, scales)     bf16 x, e4m3fn W, float32 scales[1]
    skinny_gemm_a8w8_block(x, W, x_scales, w_scales)
    skinny_gemm_a8w8_block_quant(x, W, w_scales)   bf16 x quantised in the call
each returning y [M, N] bf16 (or writing into ``y=``).
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

__all__ = [
    "SkinnyGemmError", "lib_path", "load", "OPS",
    "skinny_gemm_bf16", "skinny_gemm_gated", "skinny_gemm_fp8_tensor", "skinny_gemm_a8w8_block",
    "skinny_gemm_a8w8_block_quant",
    "skinny_gemm_run_variant", "skinny_gemm_query", "skinny_gemm_load_table", "skinny_gemm_load_table_as",
    "skinny_gemm_identity", "skinny_gemm_table_status", "skinny_gemm_num_variants",
    "skinny_gemm_variant_name", "skinny_gemm_variant_supports", "variants", "default_table_path",
]

OPS = {"bf16": 0, "gated": 1, "fp8_tensor": 2, "a8w8_block": 3, "a8w8_quant": 4}
_STATUS = {0: "OK", 1: "EINVAL", 2: "EUNSUPPORTED", 3: "ELAUNCH", 4: "ETABLE"}

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB = None
_LOCK = threading.Lock()


def lib_path() -> str:
    return os.path.join(_PKG, "libskinny_gemm.so")


def default_table_path(arch: str = "gfx950") -> str:
    """Where the library looks for this architecture's dispatch table."""
    return os.path.join(_PKG, "configs", arch, "skinny_gemm.json")


class SkinnyGemmError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


def load() -> ctypes.CDLL:
    """Load the built library (raises if it has not been built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    with _LOCK:
        if _LIB is not None:
            return _LIB
        p = lib_path()
        if not os.path.exists(p):
            raise RuntimeError(f"{p} is missing: build it with `python -m gemv_skinny_gemm_02_amd.build`"
                               " (there is no fallback path)")
        lib = ctypes.CDLL(p)
        vp, i, fp = ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p
        for name in ("skinny_gemm_bf16", "skinny_gemm_gated", "skinny_gemm_fp8_tensor"):
            f = getattr(lib, name)
            f.argtypes = [vp, vp, fp, vp, i, i, i, vp]
            f.restype = i
        lib.skinny_gemm_a8w8_block.argtypes = [vp, vp, fp, fp, vp, i, i, i, vp]
        lib.skinny_gemm_a8w8_block.restype = i
        lib.skinny_gemm_a8w8_block_quant.argtypes = [vp, vp, fp, fp, vp, i, i, i, vp]
        lib.skinny_gemm_a8w8_block_quant.restype = i
        lib.skinny_gemm_last_error.argtypes = []
        lib.skinny_gemm_last_error.restype = ctypes.c_char_p
        lib.skinny_gemm_load_table.argtypes = [ctypes.c_char_p]
        lib.skinny_gemm_load_table.restype = i
        lib.skinny_gemm_load_table_as.argtypes = [ctypes.c_char_p, ctypes.c_char_p]
        lib.skinny_gemm_load_table_as.restype = i
        lib.skinny_gemm_identity.argtypes = [ctypes.c_char_p, i]
        lib.skinny_gemm_identity.restype = i
        lib.skinny_gemm_table_status.argtypes = [ctypes.c_char_p, i]
        lib.skinny_gemm_table_status.restype = i
        lib.skinny_gemm_query.argtypes = [i, i, i, i, ctypes.c_char_p, i]
        lib.skinny_gemm_query.restype = i
        lib.skinny_gemm_num_variants.argtypes = [i]
        lib.skinny_gemm_num_variants.restype = i
        lib.skinny_gemm_variant_name.argtypes = [i, i, ctypes.c_char_p, i]
        lib.skinny_gemm_variant_name.restype = i
        lib.skinny_gemm_variant_supports.argtypes = [i, i, i]
        lib.skinny_gemm_variant_supports.restype = i
        lib.skinny_gemm_run_variant.argtypes = [i, i, vp, vp, vp, fp, fp, vp, i, i, i, vp]
        lib.skinny_gemm_run_variant.restype = i
        _LIB = lib
        return lib


def _check(st: int) -> None:
    if st != 0:
        raise SkinnyGemmError(st, load().skinny_gemm_last_error().decode(errors="replace"))


# ------------------------------------------------------------ marshalling
_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_FP8 = (torch.float8_e4m3fn, torch.uint8)


def _dev(t: torch.Tensor, name: str, dtypes, ndim: int) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, has shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a HIP device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr() if t.numel() else 0


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _out(y, M: int, N: int, like: torch.Tensor) -> torch.Tensor:
    if y is None:
        return torch.empty((M, N), dtype=torch.bfloat16, device=like.device)
    if tuple(y.shape) != (M, N):
        raise ValueError(f"y must have shape {(M, N)}, has {tuple(y.shape)}")
    return y


def _mk(x, W, rows_per_n: int):
    M, K = x.shape
    if W.shape[1] != K:
        raise ValueError(f"x is [{M}, {K}] but W has {W.shape[1]} columns")
    if W.shape[0] % rows_per_n:
        raise ValueError("gated W must have 2N rows")
    return M, W.shape[0] // rows_per_n, K


def skinny_gemm_bf16(x, W, scales=None, y=None, stream=None) -> torch.Tensor:
    """y = x . W^T with bf16 x [M,K], W [N,K]; y [M,N] bf16."""
    M, N, K = _mk(x, W, 1)
    y = _out(y, M, N, x)
    _check(load().skinny_gemm_bf16(_dev(x, "x", _BF16, 2), _dev(W, "W", _BF16, 2), None,
                                   _dev(y, "y", _BF16, 2), M, N, K, _stream(stream)))
    return y


def skinny_gemm_gated(x, W, scales=None, y=None, stream=None) -> torch.Tensor:
    """y = silu(x . Wg^T) * (x . Wu^T), W = [Wg; Wu] as one [2N, K] bf16 tensor."""
    M, N, K = _mk(x, W, 2)
    y = _out(y, M, N, x)
    _check(load().skinny_gemm_gated(_dev(x, "x", _BF16, 2), _dev(W, "W", _BF16, 2), None,
                                    _dev(y, "y", _BF16, 2), M, N, K, _stream(stream)))
    return y


def skinny_gemm_fp8_tensor(x, W, scales, y=None, stream=None) -> torch.Tensor:
    """y = scales[0] * (x . dec(W)^T); x bf16 [M,K], W e4m3fn [N,K], scales float32 [1]."""
    M, N, K = _mk(x, W, 1)
    y = _out(y, M, N, x)
    _check(load().skinny_gemm_fp8_tensor(_dev(x, "x", _BF16, 2), _dev(W, "W", _FP8, 2),
                                         _dev(scales, "scales", (torch.float32,), 1),
                                         _dev(y, "y", _BF16, 2), M, N, K, _stream(stream)))
    return y


def skinny_gemm_a8w8_block(x, W, x_scales, w_scales, y=None, stream=None) -> torch.Tensor:
    """A8W8 block scale: x e4m3fn [M,K] with x_scales [M, ceil(K/128)], W e4m3fn [N,K]
    with w_scales [ceil(N/128), ceil(K/128)]; y [M,N] bf16."""
    M, N, K = _mk(x, W, 1)
    y = _out(y, M, N, x)
    _check(load().skinny_gemm_a8w8_block(_dev(x, "x", _FP8, 2), _dev(W, "W", _FP8, 2),
                                         _dev(x_scales, "x_scales", (torch.float32,), 2),
                                         _dev(w_scales, "w_scales", (torch.float32,), 2),
                                         _dev(y, "y", _BF16, 2), M, N, K, _stream(stream)))
    return y


def skinny_gemm_a8w8_block_quant(x, W, w_scales, x_scales=None, y=None, stream=None) -> torch.Tensor:
    """A8W8 block scale with x bf16 [M,K] quantised inside the call (per row and
    128-K group, scale max|x|/448); W e4m3fn [N,K] with w_scales
    [ceil(N/128), ceil(K/128)]; y [M,N] bf16.  x_scales, if given, is a float32
    [M, ceil(K/128)] tensor that receives the scales the call used."""
    M, N, K = _mk(x, W, 1)
    y = _out(y, M, N, x)
    _check(load().skinny_gemm_a8w8_block_quant(_dev(x, "x", _BF16, 2), _dev(W, "W", _FP8, 2),
                                               _dev(w_scales, "w_scales", (torch.float32,), 2),
                                               _dev(x_scales, "x_scales", (torch.float32,), 2)
                                               if x_scales is not None else None,
                                               _dev(y, "y", _BF16, 2), M, N, K, _stream(stream)))
    return y


def skinny_gemm_run_variant(op, variant, x, W, s0=None, s1=None, y=None, stream=None) -> torch.Tensor:
    """Run one named (or numbered) variant of an op, bypassing the table."""
    opi = OPS[op] if isinstance(op, str) else int(op)
    if isinstance(variant, str):
        names = variants(opi)
        if variant not in names:
            raise ValueError(f"unknown variant {variant!r}")
        variant = names.index(variant)
    xd = _FP8 if opi == 3 else _BF16
    wd = _FP8 if opi in (2, 3, 4) else _BF16
    M, N, K = _mk(x, W, 2 if opi == 1 else 1)
    y = _out(y, M, N, x)
    p0 = _dev(s0, "s0", (torch.float32,), s0.dim()) if s0 is not None else None
    p1 = _dev(s1, "s1", (torch.float32,), s1.dim()) if s1 is not None else None
    _check(load().skinny_gemm_run_variant(opi, int(variant), None, _dev(x, "x", xd, 2), _dev(W, "W", wd, 2),
                                          p0, p1, _dev(y, "y", _BF16, 2), M, N, K, _stream(stream)))
    return y


def _text(fn, *args, size: int = 512) -> str:
    buf = ctypes.create_string_buffer(size)
    _check(fn(*args, buf, size))
    return buf.value.decode()


def skinny_gemm_query(op, M: int, N: int, K: int) -> tuple:
    """(variant name, source) that dispatch picks; source is table|default|force."""
    opi = OPS[op] if isinstance(op, str) else int(op)
    name, src = _text(load().skinny_gemm_query, opi, M, N, K).split()
    return name, src


def skinny_gemm_load_table(path: str | None = None) -> None:
    _check(load().skinny_gemm_load_table(path.encode() if path else None))


def skinny_gemm_load_table_as(path: str | None, identity: str) -> None:
    _check(load().skinny_gemm_load_table_as(path.encode() if path else None, identity.encode()))


def skinny_gemm_identity() -> str:
    return _text(load().skinny_gemm_identity)


def skinny_gemm_table_status() -> tuple:
    buf = ctypes.create_string_buffer(1024)
    engaged = load().skinny_gemm_table_status(buf, 1024)
    return bool(engaged), buf.value.decode()


def skinny_gemm_num_variants(op) -> int:
    return load().skinny_gemm_num_variants(OPS[op] if isinstance(op, str) else int(op))


def skinny_gemm_variant_name(op, i: int) -> str:
    return _text(load().skinny_gemm_variant_name, OPS[op] if isinstance(op, str) else int(op), i)


def skinny_gemm_variant_supports(op, i: int, M: int) -> bool:
    return bool(load().skinny_gemm_variant_supports(OPS[op] if isinstance(op, str) else int(op), i, M))


def variants(op=0) -> list:
    return [skinny_gemm_variant_name(op, i) for i in range(skinny_gemm_num_variants(op))]

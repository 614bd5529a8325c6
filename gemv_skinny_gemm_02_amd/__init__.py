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

Variants that split K across workgroups need a split-K workspace: device
memory the caller registers once, per stream (skinny_gemm_set_workspace) or
per device (skinny_gemm_set_device_workspace); skinny_gemm_workspace_bytes
says how much a call needs.  The binding keeps every workspace tensor it
registered alive until the process ends, so that graphs captured with it stay
valid.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

__all__ = [
    "SkinnyGemmError", "lib_path", "load", "OPS", "BUCKETS",
    "skinny_gemm_bf16", "skinny_gemm_gated", "skinny_gemm_fp8_tensor", "skinny_gemm_a8w8_block",
    "skinny_gemm_a8w8_block_quant",
    "PackedWeight", "skinny_gemm_packed_weight_bytes", "skinny_gemm_pack_weight", "skinny_gemm_bf16_packed",
    "skinny_gemm_gated_packed", "skinny_gemm_fp8_tensor_packed", "skinny_gemm_a8w8_block_packed",
    "skinny_gemm_a8w8_block_quant_packed",
    "skinny_gemm_run_variant", "skinny_gemm_query", "skinny_gemm_load_table", "skinny_gemm_load_table_as",
    "skinny_gemm_identity", "skinny_gemm_table_status", "skinny_gemm_num_variants",
    "skinny_gemm_variant_name", "skinny_gemm_variant_supports", "variants", "default_table_path",
    "skinny_gemm_calib_read", "skinny_gemm_calib_mfma", "CALIB_MFMA_FLOPS_PER_ITER_WG",
    "skinny_gemm_workspace_bytes", "skinny_gemm_variant_workspace_bytes", "skinny_gemm_set_workspace",
    "skinny_gemm_set_device_workspace", "skinny_gemm_run_static", "skinny_gemm_static_scratch_bytes",
]

# Rows buckets of dispatch (the library's list): M rounds up to the next one;
# M above the last uses the untuned tile default.
BUCKETS = (1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 64, 96, 128, 144, 160, 176, 192, 208, 224, 240, 256,
           288, 320, 352, 384, 416, 448, 480, 512)
OPS = {"bf16": 0, "gated": 1, "fp8_tensor": 2, "a8w8_block": 3, "a8w8_quant": 4,
       "bf16_packed": 5, "gated_packed": 6, "fp8_tensor_packed": 7, "a8w8_block_packed": 8, "a8w8_quant_packed": 9}
PACKED = 5            # op id offset of the forms that take a fragment-packed weight
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
        for name in ("skinny_gemm_bf16_packed", "skinny_gemm_gated_packed", "skinny_gemm_fp8_tensor_packed"):
            f = getattr(lib, name)
            f.argtypes = [vp, vp, fp, vp, i, i, i, vp]
            f.restype = i
        for name in ("skinny_gemm_a8w8_block_packed", "skinny_gemm_a8w8_block_quant_packed"):
            f = getattr(lib, name)
            f.argtypes = [vp, vp, fp, fp, vp, i, i, i, vp]
            f.restype = i
        lib.skinny_gemm_packed_weight_bytes.argtypes = [i, i, i]
        lib.skinny_gemm_packed_weight_bytes.restype = ctypes.c_size_t
        lib.skinny_gemm_pack_weight.argtypes = [i, vp, vp, i, i, vp]
        lib.skinny_gemm_pack_weight.restype = i
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
        lib.skinny_gemm_calib_read.argtypes = [vp, ctypes.c_size_t, i, i, vp, vp]
        lib.skinny_gemm_calib_read.restype = i
        lib.skinny_gemm_calib_mfma.argtypes = [i, i, vp, vp]
        lib.skinny_gemm_calib_mfma.restype = i
        lib.skinny_gemm_workspace_bytes.argtypes = [i, i, i, i]
        lib.skinny_gemm_workspace_bytes.restype = ctypes.c_size_t
        lib.skinny_gemm_variant_workspace_bytes.argtypes = [i, i, i, i]
        lib.skinny_gemm_variant_workspace_bytes.restype = ctypes.c_size_t
        lib.skinny_gemm_set_workspace.argtypes = [vp, vp, ctypes.c_size_t]
        lib.skinny_gemm_set_workspace.restype = i
        lib.skinny_gemm_set_device_workspace.argtypes = [vp, ctypes.c_size_t, vp]
        lib.skinny_gemm_set_device_workspace.restype = i
        lib.skinny_gemm_run_static.argtypes = [i, vp, vp, fp, fp, vp, i, i, i, vp]
        lib.skinny_gemm_run_static.restype = i
        lib.skinny_gemm_static_scratch_bytes.argtypes = []
        lib.skinny_gemm_static_scratch_bytes.restype = ctypes.c_size_t
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


_RAW_STREAM = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream) -> int:
    """The HIP stream handle of `stream`, default torch's current stream (read
    without building a Stream object: this runs on every call)."""
    if stream is None:
        if _RAW_STREAM is not None:
            return _RAW_STREAM(torch.cuda.current_device())
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


# ------------------------------------------------------ packed weights
_BASE_NAMES = ("bf16", "gated", "fp8_tensor", "a8w8_block", "a8w8_quant")


class PackedWeight:
    """A weight in the fragment-packed layout, as skinny_gemm_pack_weight writes
    it for one form `op` (a row-major form name) and shape: N output rows (per
    half for the gated form) and K columns.  `data` is the uint8 device tensor
    that holds it."""

    def __init__(self, data: torch.Tensor, op: str, N: int, K: int):
        self.data, self.op, self.N, self.K = data, op, N, K

    def __repr__(self) -> str:
        return f"PackedWeight(op={self.op!r}, N={self.N}, K={self.K}, bytes={self.data.numel()})"


def _base(op) -> int:
    opi = OPS[op] if isinstance(op, str) else int(op)
    return opi - PACKED if opi >= PACKED else opi


def skinny_gemm_packed_weight_bytes(op, N: int, K: int) -> int:
    """Bytes of the packed weight of form `op` at N rows (per half for gated), K columns."""
    return int(load().skinny_gemm_packed_weight_bytes(_base(op), N, K))


def skinny_gemm_pack_weight(op, W, stream=None) -> PackedWeight:
    """Write the fragment-packed copy of the row-major weight W for form `op`
    (W as that form's row-major entry point takes it) into a new device tensor."""
    b = _base(op)
    wd = _FP8 if b in (2, 3, 4) else _BF16
    rows, K = W.shape
    N = rows // 2 if b == 1 else rows
    if b == 1 and rows % 2:
        raise ValueError("gated W must have 2N rows")
    data = torch.empty(max(skinny_gemm_packed_weight_bytes(b, N, K), 0), dtype=torch.uint8, device=W.device)
    _check(load().skinny_gemm_pack_weight(b, _dev(W, "W", wd, 2), data.data_ptr() if data.numel() else 0, N, K,
                                          _stream(stream)))
    return PackedWeight(data, _BASE_NAMES[b], N, K)


def _pk(x, Wp, op: str):
    if not isinstance(Wp, PackedWeight):
        raise TypeError("W_packed must be a PackedWeight from skinny_gemm_pack_weight")
    if Wp.op != op:
        raise ValueError(f"W_packed was packed for {Wp.op!r}, not {op!r}")
    M, K = x.shape
    if Wp.K != K:
        raise ValueError(f"x is [{M}, {K}] but W_packed has K={Wp.K}")
    return M, Wp.N, K, _dev(Wp.data, "W_packed", (torch.uint8,), 1)


def skinny_gemm_bf16_packed(x, W_packed, scales=None, y=None, stream=None) -> torch.Tensor:
    """skinny_gemm_bf16 with the weight packed by skinny_gemm_pack_weight("bf16", W)."""
    M, N, K, wp = _pk(x, W_packed, "bf16")
    y = _out(y, M, N, x)
    _check(load().skinny_gemm_bf16_packed(_dev(x, "x", _BF16, 2), wp, None, _dev(y, "y", _BF16, 2), M, N, K,
                                          _stream(stream)))
    return y


def skinny_gemm_gated_packed(x, W_packed, scales=None, y=None, stream=None) -> torch.Tensor:
    """skinny_gemm_gated with the weight packed by skinny_gemm_pack_weight("gated", W)."""
    M, N, K, wp = _pk(x, W_packed, "gated")
    y = _out(y, M, N, x)
    _check(load().skinny_gemm_gated_packed(_dev(x, "x", _BF16, 2), wp, None, _dev(y, "y", _BF16, 2), M, N, K,
                                           _stream(stream)))
    return y


def skinny_gemm_fp8_tensor_packed(x, W_packed, scales, y=None, stream=None) -> torch.Tensor:
    """skinny_gemm_fp8_tensor with the weight packed by skinny_gemm_pack_weight("fp8_tensor", W)."""
    M, N, K, wp = _pk(x, W_packed, "fp8_tensor")
    y = _out(y, M, N, x)
    _check(load().skinny_gemm_fp8_tensor_packed(_dev(x, "x", _BF16, 2), wp,
                                                _dev(scales, "scales", (torch.float32,), 1),
                                                _dev(y, "y", _BF16, 2), M, N, K, _stream(stream)))
    return y


def skinny_gemm_a8w8_block_packed(x, W_packed, x_scales, w_scales, y=None, stream=None) -> torch.Tensor:
    """skinny_gemm_a8w8_block with the weight packed by skinny_gemm_pack_weight("a8w8_block", W)."""
    M, N, K, wp = _pk(x, W_packed, "a8w8_block")
    y = _out(y, M, N, x)
    _check(load().skinny_gemm_a8w8_block_packed(_dev(x, "x", _FP8, 2), wp,
                                                _dev(x_scales, "x_scales", (torch.float32,), 2),
                                                _dev(w_scales, "w_scales", (torch.float32,), 2),
                                                _dev(y, "y", _BF16, 2), M, N, K, _stream(stream)))
    return y


def skinny_gemm_a8w8_block_quant_packed(x, W_packed, w_scales, x_scales=None, y=None, stream=None) -> torch.Tensor:
    """skinny_gemm_a8w8_block_quant with the weight packed by skinny_gemm_pack_weight("a8w8_quant", W)."""
    M, N, K, wp = _pk(x, W_packed, "a8w8_quant")
    y = _out(y, M, N, x)
    _check(load().skinny_gemm_a8w8_block_quant_packed(_dev(x, "x", _BF16, 2), wp,
                                                      _dev(w_scales, "w_scales", (torch.float32,), 2),
                                                      _dev(x_scales, "x_scales", (torch.float32,), 2)
                                                      if x_scales is not None else None,
                                                      _dev(y, "y", _BF16, 2), M, N, K, _stream(stream)))
    return y


def skinny_gemm_run_variant(op, variant, x, W, s0=None, s1=None, y=None, stream=None) -> torch.Tensor:
    """Run one named (or numbered) variant of an op, bypassing the table.  For a
    packed op W is the PackedWeight of its row-major form."""
    opi = OPS[op] if isinstance(op, str) else int(op)
    if isinstance(variant, str):
        names = variants(opi)
        if variant not in names:
            raise ValueError(f"unknown variant {variant!r}")
        variant = names.index(variant)
    b = _base(opi)
    xd = _FP8 if b == 3 else _BF16
    wd = _FP8 if b in (2, 3, 4) else _BF16
    if opi >= PACKED:
        M, N, K, wp = _pk(x, W, _BASE_NAMES[b])
    else:
        M, N, K = _mk(x, W, 2 if b == 1 else 1)
        wp = _dev(W, "W", wd, 2)
    y = _out(y, M, N, x)
    p0 = _dev(s0, "s0", (torch.float32,), s0.dim()) if s0 is not None else None
    p1 = _dev(s1, "s1", (torch.float32,), s1.dim()) if s1 is not None else None
    _check(load().skinny_gemm_run_variant(opi, int(variant), None, _dev(x, "x", xd, 2), wp,
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


# ------------------------------------------------------ split-K workspace
# Every workspace tensor registered through the binding stays alive until the
# process ends, also after another one replaces it: a graph captured while it
# was registered keeps its address.  Register a workspace once per stream (or
# device) and reuse it, rather than registering a new one per call.
_HELD = []


def _opi(op) -> int:
    return OPS[op] if isinstance(op, str) else int(op)


def skinny_gemm_workspace_bytes(op, M: int, N: int, K: int) -> int:
    """Bytes of split-K workspace the call (op, M, N, K) needs under the
    current dispatch (0 if none)."""
    return int(load().skinny_gemm_workspace_bytes(_opi(op), M, N, K))


def skinny_gemm_variant_workspace_bytes(op, variant, M: int, N: int) -> int:
    """Bytes of split-K workspace one variant needs at M rows and N outputs."""
    if isinstance(variant, str):
        variant = variants(op).index(variant)
    return int(load().skinny_gemm_variant_workspace_bytes(_opi(op), int(variant), M, N))


def _ws_tensor(ws, device):
    if ws is None:
        return None
    if isinstance(ws, int):
        n = max(int(ws), 256 << 10)
        ws = torch.empty((n + 255) // 256 * 256, dtype=torch.uint8, device=device)
    if not isinstance(ws, torch.Tensor) or not ws.is_cuda or not ws.is_contiguous():
        raise ValueError("a workspace is a byte count or a contiguous device tensor")
    return ws


def skinny_gemm_set_workspace(ws, stream=None) -> torch.Tensor | None:
    """Register a split-K workspace for the calls on `stream` (default: the
    current stream): a device tensor, or a byte count to allocate one of;
    None removes the stream's registration.  Returns the tensor."""
    t = _ws_tensor(ws, torch.device("cuda", torch.cuda.current_device()))
    _check(load().skinny_gemm_set_workspace(_stream(stream), t.data_ptr() if t is not None else None,
                                            t.numel() * t.element_size() if t is not None else 0))
    if t is not None:
        _HELD.append(t)
    return t


def skinny_gemm_set_device_workspace(ws, stream=None) -> torch.Tensor | None:
    """Register the current device's split-K workspace (used by every stream
    without one of its own): a device tensor, or a byte count to allocate one
    of; None removes it.  Its counters are cleared on `stream` (default: the
    current stream), which is synchronised before returning so that calls on
    any stream see them cleared.  Returns the tensor."""
    t = _ws_tensor(ws, torch.device("cuda", torch.cuda.current_device()))
    _check(load().skinny_gemm_set_device_workspace(t.data_ptr() if t is not None else None,
                                                   t.numel() * t.element_size() if t is not None else 0,
                                                   _stream(stream)))
    if t is not None:
        _HELD.append(t)
        torch.cuda.synchronize()
    return t


def skinny_gemm_static_scratch_bytes() -> int:
    """Bytes of split-K partials the library's static device scratch holds."""
    return int(load().skinny_gemm_static_scratch_bytes())


def skinny_gemm_run_static(op, x, W, s0=None, s1=None, y=None, stream=None) -> torch.Tensor:
    """The op's entry point with its split-K partials in the library's static
    device scratch: allocates nothing on the device and needs no workspace
    (calls that overlap in time on one device race on the scratch).  Scale
    arrays as skinny_gemm_run_variant; for a packed op W is its
    PackedWeight."""
    opi = _opi(op)
    b = _base(opi)
    xd = _FP8 if b == 3 else _BF16
    wd = _FP8 if b in (2, 3, 4) else _BF16
    if opi >= PACKED:
        M, N, K, wp = _pk(x, W, _BASE_NAMES[b])
    else:
        M, N, K = _mk(x, W, 2 if b == 1 else 1)
        wp = _dev(W, "W", wd, 2)
    y = _out(y, M, N, x)
    p0 = _dev(s0, "s0", (torch.float32,), s0.dim()) if s0 is not None else None
    p1 = _dev(s1, "s1", (torch.float32,), s1.dim()) if s1 is not None else None
    _check(load().skinny_gemm_run_static(opi, _dev(x, "x", xd, 2), wp, p0, p1, _dev(y, "y", _BF16, 2), M, N, K,
                                         _stream(stream)))
    return y


# ------------------------------------------------------ measurement helpers
CALIB_MFMA_FLOPS_PER_ITER_WG = 4 * 8 * 32768   # 4 waves x 8 MFMA 32x32x16 per round


def _sink(sink, like_device):
    if sink is None:
        sink = torch.empty(256, dtype=torch.int32, device=like_device)
    if sink.dtype != torch.int32 or sink.numel() < 256 or not sink.is_cuda or not sink.is_contiguous():
        raise ValueError("sink must be a contiguous int32 device tensor of at least 256 words")
    return sink


def skinny_gemm_calib_read(buf: torch.Tensor, grid: int, sink=None, stream=None, sweep: bool = False) -> None:
    """Read every byte of the contiguous device tensor `buf` once with `grid`
    workgroups, a slice each or (sweep) all together (a measurement kernel: it
    computes nothing of the linear)."""
    if not isinstance(buf, torch.Tensor) or not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    sink = _sink(sink, buf.device)
    _check(load().skinny_gemm_calib_read(buf.data_ptr(), buf.numel() * buf.element_size(), int(grid),
                                         1 if sweep else 0, sink.data_ptr(), _stream(stream)))


def skinny_gemm_calib_mfma(grid: int, iters: int, sink=None, stream=None) -> int:
    """Run grid * iters rounds of 4 waves x 8 bf16 MFMA (a measurement kernel);
    returns the flops it issues."""
    sink = _sink(sink, torch.device("cuda", torch.cuda.current_device()))
    _check(load().skinny_gemm_calib_mfma(int(grid), int(iters), sink.data_ptr(), _stream(stream)))
    return int(grid) * int(iters) * CALIB_MFMA_FLOPS_PER_ITER_WG

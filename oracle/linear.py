"""The four forms of the skinny decode linear, as plain float64 definitions.
Test infrastructure only.

All inputs are raw bits as numpy arrays (bf16 as uint16, e4m3fn as uint8) and
float32 scales.  x is [M, K] row-major, W is [N, K] row-major (one output
column per row of W), y is [M, N].  Every function takes an optional ``cols``:
an index array of output columns to compute, so that a full-size problem can be
spot-checked column by column; the result then has shape [M, len(cols)].

The product of the decoded arrays is a library matmul in float64.  The inputs
are exact in float64 (bf16 and e4m3fn values, and the product of an e4m3fn value
with an fp32 scale, fit in 53 bits), so the only rounding is float64
accumulation, about K * 2^-53 relative.
"""
from __future__ import annotations

import numpy as np

from .formats import dec_bf16, dec_e4m3fn, silu

BLOCK = 128          # scale block edge: 1 x 128 for x, 128 x 128 for W
_ROWS = 8192         # rows of W decoded at a time (memory only; no reordering)


def _cols(n: int, cols):
    return np.arange(n, dtype=np.int64) if cols is None else np.asarray(cols, dtype=np.int64)


def _matmul_rows(xd: np.ndarray, w_rows_fn, cols: np.ndarray) -> np.ndarray:
    """y[:, j] = xd . dec(W[cols[j]])  for the given columns, decoding W in
    bounded pieces.  ``w_rows_fn(idx)`` returns the decoded float64 rows."""
    y = np.empty((xd.shape[0], cols.size), dtype=np.float64)
    for lo in range(0, cols.size, _ROWS):
        idx = cols[lo:lo + _ROWS]
        y[:, lo:lo + idx.size] = xd @ w_rows_fn(idx).T
    return y


def linear_bf16(x, w, cols=None) -> np.ndarray:
    """y[m, n] = sum_k x[m, k] W[n, k], bf16 inputs (mstar PR #1104, "Why":
    the decode linears routed between skinny GEMM, GEMV and hipBLASLt)."""
    xd = dec_bf16(x)
    return _matmul_rows(xd, lambda idx: dec_bf16(w[idx]), _cols(w.shape[0], cols))


def linear_gated(x, w, cols=None) -> np.ndarray:
    """Fused gate/up: W is one [2N, K] buffer, gate rows [0, N), up rows
    [N, 2N); y[m, n] = silu(g[m, n]) * u[m, n] with g = x Wg^T and u = x Wu^T
    (mstar PR #1104, "Why" -- decode_gemv_silu_mul -- and "What changed" -- the
    fused gate/up's own gated1- table entry).  g and u are not rounded."""
    n2 = w.shape[0]
    if n2 % 2:
        raise ValueError("gated W must have an even number of rows [2N, K]")
    N = n2 // 2
    c = _cols(N, cols)
    xd = dec_bf16(x)
    g = _matmul_rows(xd, lambda idx: dec_bf16(w[idx]), c)
    u = _matmul_rows(xd, lambda idx: dec_bf16(w[idx + N]), c)
    return silu(g) * u


def linear_fp8_tensor(x, wq, w_scale, cols=None) -> np.ndarray:
    """y = s * (x . dec(Wq)^T) with bf16 x, e4m3fn Wq and one fp32 scale s for
    the whole weight (mstar PR #1102, "What changed": an fp8 copy of the draft
    head with a single scale)."""
    s = float(np.asarray(w_scale, dtype=np.float32).reshape(-1)[0])
    xd = dec_bf16(x)
    return s * _matmul_rows(xd, lambda idx: dec_e4m3fn(wq[idx]), _cols(wq.shape[0], cols))


def dequant_a8w8(xq, xs, wq, ws, cols=None):
    """Exact float64 dequantisation of the A8W8 block-scale operands:
    x~[m, k] = xs[m, k // 128] * dec(xq[m, k]) and
    W~[n, k] = ws[n // 128, k // 128] * dec(wq[n, k]).  A partial last group or
    block uses its own scale.  Returns (x~, W~[cols])."""
    M, K = xq.shape
    c = _cols(wq.shape[0], cols)
    kgrp = np.arange(K) // BLOCK
    xs64 = np.asarray(xs, dtype=np.float64)
    ws64 = np.asarray(ws, dtype=np.float64)
    xd = dec_e4m3fn(xq) * xs64[:, kgrp]
    wd = dec_e4m3fn(wq[c]) * ws64[(c // BLOCK)[:, None], kgrp[None, :]]
    return xd, wd


def linear_a8w8_block(xq, xs, wq, ws, cols=None) -> np.ndarray:
    """A8W8 block-scale linear (Decode optimization round 3, "Retained
    change 2"): fp8 activations with one fp32 scale per row per 128 K-columns,
    fp8 weights with one fp32 scale per 128 x 128 block; y = x~ . W~^T over the
    dequantised operands (see ``dequant_a8w8``)."""
    c = _cols(wq.shape[0], cols)
    y = np.empty((xq.shape[0], c.size), dtype=np.float64)
    for lo in range(0, c.size, _ROWS):
        xd, wd = dequant_a8w8(xq, xs, wq, ws, c[lo:lo + _ROWS])
        y[:, lo:lo + wd.shape[0]] = xd @ wd.T
    return y

"""Activation quantisation for A8W8, decided in float32.  Test infrastructure only.

The A8W8 block-scale form takes x as OCP e4m3fn codes with one float32 scale
per row and 128-K group (Decode optimization round 3, "Retained change 2").
The quantisation that produces them runs as its own kernels upstream of the
linear there: the profile of that page ("Profiling: why M=1-8 decode is
dispatch-bound") counts the dynamic-quant launches among the launch-floor
bound ones, and its "Rejected paths" section leaves folding the quantisation
into the GEMM as open work.

Reading taken, since the pages do not print the quantiser: for every row m and
group g of 128 consecutive K (the last group may be shorter)

    a      = max |x[m, k]|                 over k in the group (exact)
    s      = a / 448  in float32           (IEEE division, round to nearest
                                            even); s = 1 when a = 0
    q[m,k] = e4m3fn(RNE(clamp(x[m,k] / s, -448, 448)))
             where x / s is one float32 division and RNE rounds that float32
             value once to the e4m3fn grid

448 is the largest finite e4m3fn magnitude.  Because every quantity that
decides a code is a float32 result of one correctly rounded operation, the
codes and scales here are bit-exact targets for any implementation that uses
the same operations.
"""
from __future__ import annotations

import numpy as np

from .formats import E4M3FN_TABLE, dec_bf16
from .linear import BLOCK, linear_a8w8_block

E4M3_MAX = 448.0

# value -> code for the 127 non-negative finite codes (0x00 .. 0x7E)
_POS_VALUES = E4M3FN_TABLE[:0x7F].copy()
assert np.all(np.diff(_POS_VALUES) > 0)


def e4m3fn_rne_bits(v) -> np.ndarray:
    """float64 values (finite) -> OCP e4m3fn codes: clamp to [-448, 448], then
    one round-to-nearest-even step onto the e4m3fn grid (4 significant bits
    from 2^-6 up, the fixed quantum 2^-9 below)."""
    v = np.clip(np.asarray(v, dtype=np.float64), -E4M3_MAX, E4M3_MAX)
    a = np.abs(v)
    mant, ex = np.frexp(a)                              # a = mant * 2^ex, mant in [0.5, 1)
    q_norm = np.ldexp(np.rint(np.ldexp(mant, 4)), ex - 4)
    q_sub = np.rint(a * 2.0 ** 9) * 2.0 ** -9
    q = np.where(a >= 2.0 ** -6, q_norm, q_sub)
    idx = np.searchsorted(_POS_VALUES, q)
    if not np.all(_POS_VALUES[np.minimum(idx, 126)] == q):
        raise AssertionError("rounded value off the e4m3fn grid")
    code = idx.astype(np.uint8)
    return np.where((v < 0) & (code != 0), code | np.uint8(0x80), code).astype(np.uint8)


def quantize_a8w8_x(x_bits, block: int = BLOCK):
    """bf16 x [M, K] (bit patterns) -> (e4m3fn codes [M, K] uint8, float32
    scales [M, ceil(K/block)]), by the reading in the module header."""
    x32 = dec_bf16(x_bits).astype(np.float32)          # exact
    M, K = x32.shape
    G = -(-K // block)
    codes = np.empty((M, K), dtype=np.uint8)
    scales = np.empty((M, G), dtype=np.float32)
    for g in range(G):
        blk = x32[:, g * block:(g + 1) * block]
        a = np.max(np.abs(blk), axis=1) if blk.size else np.zeros(M, np.float32)
        s = np.where(a > 0, a / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
        r = (blk / s[:, None]).astype(np.float32)      # one float32 division per element
        codes[:, g * block:(g + 1) * block] = e4m3fn_rne_bits(r.astype(np.float64))
        scales[:, g] = s
    return codes, scales


def linear_a8w8_quant(x_bits, wq, ws, cols=None):
    """A8W8 block scale with the activation quantised inside: returns
    (y float64 [M, len(cols)], codes, x scales)."""
    codes, xs = quantize_a8w8_x(x_bits)
    return linear_a8w8_block(codes, xs, wq, ws, cols), codes, xs

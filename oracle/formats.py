"""Storage formats, decoded exactly into float64.  Test infrastructure only.

bf16: the upper 16 bits of an IEEE-754 binary32 (1 sign, 8 exponent, 7
fraction bits).  Every bf16 value is a float32 value, hence exact in float64.

OCP e4m3fn (OCP 8-bit Floating Point Specification, E4M3 encoding): 1 sign,
4 exponent (bias 7), 3 fraction bits; no infinities; S.1111.111 is NaN; the
largest finite magnitude is 1.75 * 2^8 = 448; exponent field 0 encodes
subnormals m * 2^-9.  The configurations quantise with scale = amax/448, which
is this encoding's finite maximum.
"""
from __future__ import annotations

import math

import numpy as np


def dec_bf16(bits) -> np.ndarray:
    """bf16 bit patterns (any integer dtype, 16 significant bits) -> float64."""
    b = np.asarray(bits).astype(np.uint32) & np.uint32(0xFFFF)
    with np.errstate(invalid="ignore"):          # NaN payloads cast quietly
        return (b << np.uint32(16)).view(np.float32).astype(np.float64)


def _e4m3fn_value(code: int) -> float:
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return s * m * 2.0 ** -9            # subnormal: 0.mmm * 2^(1-7)
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3FN_TABLE = np.array([_e4m3fn_value(c) for c in range(256)], dtype=np.float64)
E4M3FN_TABLE.setflags(write=False)


def dec_e4m3fn(codes) -> np.ndarray:
    """OCP e4m3fn bytes -> float64 (NaN codes decode to NaN)."""
    return E4M3FN_TABLE[np.asarray(codes).astype(np.uint8)]


def bf16_rne_bits(v) -> np.ndarray:
    """float64 -> bf16 bits with one round-to-nearest-even step.

    Rounds the value itself to 8 significant bits (not through float32, which
    would round twice).  Magnitudes at or above the bf16 overflow threshold
    become infinity; the subnormal range uses the fixed quantum 2^-133.
    """
    v = np.asarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.float64)
    mant, ex = np.frexp(v)                           # v = mant * 2^ex, |mant| in [0.5, 1)
    normal = np.abs(v) >= 2.0 ** -126
    q_norm = np.ldexp(np.rint(np.ldexp(mant, 8)), ex - 8)
    q_sub = np.rint(v * 2.0 ** 133) * 2.0 ** -133
    out[...] = np.where(normal, q_norm, q_sub)
    out = np.where(np.isnan(v), np.nan, out)
    with np.errstate(over="ignore"):
        f = out.astype(np.float32)                   # exact: out has <= 8 significant bits
    f = np.where(np.abs(out) >= 2.0 ** 128, np.copysign(np.float32(np.inf), out), f)
    return (np.ascontiguousarray(f, dtype=np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def silu(g) -> np.ndarray:
    """SiLU in float64, g * sigmoid(g), in the overflow-free form:
    g / (1 + e^-g) for g >= 0 and g e^g / (1 + e^g) for g < 0."""
    g = np.asarray(g, dtype=np.float64)
    out = np.empty_like(g)
    pos = g >= 0
    out[pos] = g[pos] / (1.0 + np.exp(-g[pos]))
    eg = np.exp(g[~pos])
    out[~pos] = g[~pos] * eg / (1.0 + eg)
    return out

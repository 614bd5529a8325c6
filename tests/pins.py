"""Pins for the oracle's four linear forms, written against an implementation
passed in, so that the same checks can be shown to catch planted mistakes.

Each ``pins_*`` returns a list of failure strings (empty: every pin holds).
The pins use: brute force in exact rational arithmetic on tiny shapes; one-hot
and identity inputs, which expose a transposed or mis-indexed operand exactly;
exact power-of-two scaling invariants; high-precision decimal SiLU.
"""
from __future__ import annotations

import decimal
from fractions import Fraction

import numpy as np

from oracle.formats import dec_bf16, dec_e4m3fn

U = 2.0 ** -53


def _fr(a):
    return [[Fraction(float(v)) for v in row] for row in np.asarray(a, np.float64)]


def _exact_mm(xd, wd):
    X, W = _fr(xd), _fr(wd)
    return [[sum((a * b for a, b in zip(xr, wr)), Fraction(0)) for wr in W] for xr in X]


def _bound(xd, wd):
    K = xd.shape[1]
    return 2 * K * U * (np.abs(xd) @ np.abs(wd).T) + 1e-300


def _bf16_from(r, shape, std=1.0):
    v = (r.standard_normal(shape) * std).astype(np.float32)
    return (v.view(np.uint32) >> 16).astype(np.uint16)     # truncation is fine for test data


def _fp8_from(r, shape):
    codes = r.integers(0, 256, size=shape).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38                   # no NaN codes
    return codes


def _check_close(name, got, exact, bound, fails):
    got = np.asarray(got, np.float64)
    ex = np.array([[float(v) for v in row] for row in exact])
    if got.shape != ex.shape:
        fails.append(f"{name}: shape {got.shape} != {ex.shape}")
        return
    err = np.abs(got - ex)
    if not np.all(err <= bound):
        fails.append(f"{name}: max err {err.max():.3e} > bound")


# ----------------------------------------------------------------- bf16 form
def pins_bf16(fn) -> list:
    fails = []
    r = np.random.default_rng(11)
    for (M, N, K) in [(1, 3, 5), (3, 4, 7), (2, 5, 16), (4, 2, 33)]:
        x, w = _bf16_from(r, (M, K)), _bf16_from(r, (N, K), 0.05)
        xd, wd = dec_bf16(x), dec_bf16(w)
        _check_close(f"bf16 brute {M}x{N}x{K}", fn(x, w), _exact_mm(xd, wd), _bound(xd, wd), fails)
    # one-hot rows of x pick columns of W exactly: y[m, n] = W[n, k_m]
    M, N, K = 3, 6, 10
    w = _bf16_from(r, (N, K))
    x = np.zeros((M, K), np.uint16)
    ks = [0, 7, 9]
    for m, k in enumerate(ks):
        x[m, k] = 0x3F80                                    # 1.0
    y = np.asarray(fn(x, w))
    want = dec_bf16(w)[:, ks].T
    if y.shape != want.shape or not np.array_equal(y, want):
        fails.append("bf16 one-hot: y[m, n] != W[n, k_m]")
    # identity W (N = K) gives y = x
    K = 8
    x = _bf16_from(r, (2, K))
    eye = np.zeros((K, K), np.uint16)
    eye[np.arange(K), np.arange(K)] = 0x3F80
    if not np.array_equal(np.asarray(fn(x, eye)), dec_bf16(x)):
        fails.append("bf16 identity: y != x")
    # exact scaling by 2 (exponent shift) doubles y exactly
    x, w = _bf16_from(r, (2, 9)), _bf16_from(r, (4, 9))
    x2 = (x.astype(np.uint32) + (1 << 7)).astype(np.uint16)  # exponent + 1 (no zeros/infs here)
    if not np.array_equal(np.asarray(fn(x2, w)), 2 * np.asarray(fn(x, w))):
        fails.append("bf16 scaling: y(2x) != 2 y(x)")
    # cols selects output columns
    x, w = _bf16_from(r, (2, 12)), _bf16_from(r, (9, 12))
    full = np.asarray(fn(x, w))
    cols = np.array([0, 4, 8])
    if not np.array_equal(np.asarray(fn(x, w, cols=cols)), full[:, cols]):
        fails.append("bf16 cols: subset differs from full")
    return fails


# ---------------------------------------------------------------- gated form
def _silu_dec(g: Fraction) -> decimal.Decimal:
    with decimal.localcontext() as ctx:
        ctx.prec = 50
        gd = decimal.Decimal(g.numerator) / decimal.Decimal(g.denominator)
        return gd / (1 + (-gd).exp())


def pins_gated(fn) -> list:
    fails = []
    r = np.random.default_rng(12)
    for (M, N, K) in [(1, 3, 6), (2, 4, 9), (3, 2, 16)]:
        x = _bf16_from(r, (M, K))
        w = _bf16_from(r, (2 * N, K), 0.3)
        xd, wd = dec_bf16(x), dec_bf16(w)
        G, Uu = _exact_mm(xd, wd[:N]), _exact_mm(xd, wd[N:])
        want = np.array([[float(_silu_dec(G[m][n]) * decimal.Decimal(Uu[m][n].numerator)
                                / decimal.Decimal(Uu[m][n].denominator))
                          for n in range(N)] for m in range(M)])
        got = np.asarray(fn(x, w), np.float64)
        if got.shape != want.shape or not np.allclose(got, want, rtol=1e-12, atol=1e-14):
            fails.append(f"gated brute {M}x{N}x{K}")
    # one-hot: g = Wg[n, k], u = Wu[n, k]; y = silu(Wg[n,k]) * Wu[n,k]
    N, K = 4, 5
    w = np.zeros((2 * N, K), np.uint16)
    w[:N, 2] = [0x3F80, 0xBF80, 0x0000, 0x4000]             # gate column: 1, -1, 0, 2
    w[N:, 2] = [0x4000, 0x4000, 0x3F80, 0x3F00]             # up column: 2, 2, 1, 0.5
    x = np.zeros((1, K), np.uint16)
    x[0, 2] = 0x3F80
    got = np.asarray(fn(x, w), np.float64)[0]
    s1 = 0.7310585786300049                                 # e / (1 + e)
    want = np.array([2 * s1, 2 * (s1 - 1.0), 0.0, 0.5 * (2 / (1 + np.exp(-2.0)))])
    if not np.allclose(got, want, rtol=1e-15, atol=0):
        fails.append(f"gated one-hot: {got} != {want}")
    return fails


# ---------------------------------------------------------- fp8 tensor form
def pins_fp8_tensor(fn) -> list:
    fails = []
    r = np.random.default_rng(13)
    for (M, N, K) in [(1, 4, 8), (2, 3, 17), (4, 5, 32)]:
        x = _bf16_from(r, (M, K))
        wq = _fp8_from(r, (N, K))
        s = np.array([0.0371], np.float32)
        xd, wd = dec_bf16(x), dec_e4m3fn(wq) * np.float64(s[0])
        _check_close(f"fp8 brute {M}x{N}x{K}", fn(x, wq, s), _exact_mm(xd, wd), _bound(xd, wd), fails)
    # every code through a one-hot row, scale 1: y[0, c] = dec(c)
    codes = np.arange(256, dtype=np.uint8)
    codes = codes[(codes & 0x7F) != 0x7F]
    wq = np.zeros((codes.size, 3), np.uint8)
    wq[:, 1] = codes
    x = np.zeros((1, 3), np.uint16)
    x[0, 1] = 0x3F80
    got = np.asarray(fn(x, wq, np.array([1.0], np.float32)))[0]
    if not np.array_equal(got, dec_e4m3fn(codes)):
        fails.append("fp8 one-hot: y != dec(code)")
    # doubling the scale doubles y exactly
    x, wq = _bf16_from(r, (2, 16)), _fp8_from(r, (3, 16))
    a = np.asarray(fn(x, wq, np.array([0.25], np.float32)))
    b = np.asarray(fn(x, wq, np.array([0.5], np.float32)))
    if not np.array_equal(b, 2 * a):
        fails.append("fp8 scale: y(2s) != 2 y(s)")
    return fails


# ------------------------------------------------------------ A8W8 block form
def _a8w8_brute(xq, xs, wq, ws):
    M, K = xq.shape
    N = wq.shape[0]
    xdv, wdv = dec_e4m3fn(xq), dec_e4m3fn(wq)
    out, mag = [], np.zeros((M, N))
    for m in range(M):
        row = []
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                sx = Fraction(float(xs[m, k // 128]))
                sw = Fraction(float(ws[n // 128, k // 128]))
                t = sx * Fraction(float(xdv[m, k])) * sw * Fraction(float(wdv[n, k]))
                acc += t
                mag[m, n] += abs(float(t))
            row.append(acc)
        out.append(row)
    return out, 2 * K * U * mag + 1e-300


def pins_a8w8_block(fn) -> list:
    fails = []
    r = np.random.default_rng(14)
    # several blocks in both N and K, with ragged last blocks
    for (M, N, K) in [(2, 3, 40), (2, 130, 136), (1, 257, 260)]:
        xq, wq = _fp8_from(r, (M, K)), _fp8_from(r, (N, K))
        xs = r.uniform(0.5, 2.0, size=(M, -(-K // 128))).astype(np.float32)
        ws = r.uniform(0.01, 0.1, size=(-(-N // 128), -(-K // 128))).astype(np.float32)
        cols = np.array([0, 1, N - 1]) if N > 8 else None
        exact, bound = _a8w8_brute(xq, xs, wq[cols] if cols is not None else wq,
                                   ws[(cols // 128)] if cols is not None else ws)
        if cols is not None:
            # brute force was computed on the selected rows with their own block rows
            got = np.asarray(fn(xq, xs, wq, ws, cols=cols))
            # fix the brute's block-row indexing: it saw rows 0..len(cols)-1
            exact2, bound2 = [], np.zeros((M, cols.size))
            for m in range(M):
                exact2.append([])
                for j, n in enumerate(cols):
                    e, b = _a8w8_brute(xq[m:m + 1], xs[m:m + 1], wq[n:n + 1], ws[n // 128:n // 128 + 1])
                    exact2[m].append(e[0][0])
                    bound2[m, j] = b[0, 0]
            _check_close(f"a8w8 brute {M}x{N}x{K}", got, exact2, bound2, fails)
        else:
            _check_close(f"a8w8 brute {M}x{N}x{K}", fn(xq, xs, wq, ws), exact, bound, fails)
    # block-scale placement: one-hot x at column k, ws with distinct per-block
    # values -> y[0, n] = xs[0, k//128] * ws[n//128, k//128] * dec(wq[n, k])
    N, K = 384, 384
    wq = _fp8_from(r, (N, K))
    ws = (np.arange(9, dtype=np.float32).reshape(3, 3) + 1) * np.float32(0.125)
    for k in (5, 200, 383):
        xq = np.zeros((1, K), np.uint8)
        xq[0, k] = 0x38
        xs = np.array([[1.0, 2.0, 4.0]], np.float32)
        got = np.asarray(fn(xq, xs, wq, ws))[0]
        want = xs[0, k // 128] * ws[np.arange(N) // 128, k // 128] * dec_e4m3fn(wq[:, k])
        if not np.array_equal(got, want):
            fails.append(f"a8w8 one-hot block placement k={k}")
    # moving a power of two from ws to xs leaves y unchanged, exactly
    M, N, K = 2, 130, 256
    xq, wq = _fp8_from(r, (M, K)), _fp8_from(r, (N, K))
    xs = r.uniform(0.5, 2.0, size=(M, 2)).astype(np.float32)
    ws = r.uniform(0.01, 0.1, size=(2, 2)).astype(np.float32)
    a = np.asarray(fn(xq, xs, wq, ws))
    b = np.asarray(fn(xq, xs * 2, wq, ws / 2))
    if not np.array_equal(a, b):
        fails.append("a8w8 scale invariance")
    return fails

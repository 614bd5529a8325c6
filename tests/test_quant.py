"""The activation quantiser of the oracle (A8W8 with x quantised inside) against
what the e4m3fn grid and round-to-nearest-even fix, and the pins against
planted mistakes.  CPU only."""
import numpy as np
import pytest
import torch

import oracle
from oracle import formats, quant

FINITE = [c for c in range(256) if c not in (0x7F, 0xFF)]


def grid_pins(enc):
    """Mistakes found in an e4m3fn encoder `enc` (float64 array -> codes)."""
    bad = []
    # every finite code's value maps back to itself (-0 to +0)
    vals = formats.dec_e4m3fn(np.array(FINITE))
    want = np.array([c if c != 0x80 else 0 for c in FINITE], dtype=np.uint8)
    if not np.array_equal(enc(vals), want):
        bad.append("fixed points")
    # the midpoint of two neighbours goes to the one with an even fraction
    # field; a hair either side goes to the nearer one
    pos = formats.E4M3FN_TABLE[:0x7F]
    lo, hi = pos[:-1], pos[1:]
    mid = (lo + hi) / 2
    even = np.where(np.arange(126) % 2 == 0, np.arange(126), np.arange(1, 127)).astype(np.uint8)
    for sgn, flip in ((1.0, 0), (-1.0, 0x80)):
        got = enc(sgn * mid)
        exp = np.where(even == 0, 0, even | flip).astype(np.uint8)
        if not np.array_equal(got, exp):
            bad.append(f"ties sign {sgn}")
        eps = (hi - lo) * 1e-6
        if not np.array_equal(enc(sgn * (mid - eps)), np.where(np.arange(126) == 0, 0, np.arange(126) | flip).astype(np.uint8)):
            bad.append(f"below midpoint sign {sgn}")
        if not np.array_equal(enc(sgn * (mid + eps)), (np.arange(1, 127) | flip).astype(np.uint8)):
            bad.append(f"above midpoint sign {sgn}")
    # saturation at the largest finite magnitude
    if list(enc(np.array([448.0, 464.0, 476.0, 1e30, -464.0, -1e30]))) != [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]:
        bad.append("saturation")
    return bad


def quant_pins(qfn):
    """Mistakes found in a quantiser `qfn` (bf16 bits [M,K] -> codes, scales)."""
    bad = []
    r = np.random.default_rng(5)
    M, K = 6, 200                                    # groups of 128 and 72
    x = (r.standard_normal((M, K)) * np.array([1, 1e-3, 1e3, 1, 1, 1])[:, None]).astype(np.float32)
    x[3] = 0.0                                       # an all-zero row
    x[4, 128:] = 0.0                                 # a zero second group
    x[5, 7] = 3.0e4                                  # one large element
    bits = oracle.bf16_rne_bits(x.astype(np.float64))
    xv = formats.dec_bf16(bits).astype(np.float32)
    codes, s = qfn(bits)
    if s.shape != (M, 2) or s.dtype != np.float32:
        return ["scale shape"]
    for g, sl in enumerate((slice(0, 128), slice(128, 200))):
        a = np.max(np.abs(xv[:, sl]), axis=1)
        want = np.where(a > 0, a / np.float32(448.0), np.float32(1.0)).astype(np.float32)
        if not np.array_equal(s[:, g], want):
            bad.append(f"scales of group {g}")
        dv = formats.dec_e4m3fn(codes[:, sl])
        nz = a > 0
        # the group maximum lands on +-448
        if not np.all(np.max(np.abs(dv[nz]), axis=1) == 448.0):
            bad.append(f"group {g} maximum is not 448")
        if not np.all(codes[~nz, sl] == 0):
            bad.append(f"group {g} zero rows")
        # every code is the nearest grid point to x / s (half a grid step)
        with np.errstate(divide="ignore", invalid="ignore"):
            rr = (xv[:, sl] / s[:, g:g + 1]).astype(np.float64)
        step = np.where(np.abs(rr) >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(np.abs(rr), 1e-300))) - 3), 2.0 ** -9)
        if not np.all(np.abs(dv - np.clip(rr, -448, 448)) <= step / 2 + 1e-300):
            bad.append(f"group {g} rounding distance")
    # scaling x by a power of two keeps the codes and scales the scales
    # (all-zero groups keep the scale 1)
    codes2, s2 = qfn(oracle.bf16_rne_bits(xv.astype(np.float64) * 2.0 ** -5))
    zero = np.stack([np.max(np.abs(xv[:, :128]), axis=1) == 0, np.max(np.abs(xv[:, 128:]), axis=1) == 0], axis=1)
    if not (np.array_equal(codes2, codes) and np.array_equal(s2, np.where(zero, s, s * np.float32(2.0 ** -5)))):
        bad.append("power-of-two scaling")
    return bad


def test_encoder_pins():
    assert grid_pins(quant.e4m3fn_rne_bits) == []


def test_encoder_matches_torch_cast():
    """A library route: torch's float32 -> float8_e4m3fn cast rounds to nearest
    even; on values already clamped to +-448 it must agree bit for bit (zero
    magnitudes compared without their sign)."""
    r = np.random.default_rng(11)
    v = np.concatenate([r.uniform(-448, 448, 200000), r.standard_normal(200000) * 1e-2,
                        r.standard_normal(100000) * 1e-3]).astype(np.float32)
    ours = quant.e4m3fn_rne_bits(v.astype(np.float64))
    theirs = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    theirs = np.where((theirs & 0x7F) == 0, 0, theirs)
    assert np.array_equal(ours, theirs)


def test_quantiser_pins():
    assert quant_pins(quant.quantize_a8w8_x) == []


def test_linear_with_quant_is_a8w8_of_the_codes():
    r = np.random.default_rng(2)
    M, N, K = 3, 130, 256
    x = oracle.bf16_rne_bits(r.standard_normal((M, K)))
    wq = r.integers(0, 0x7E, size=(N, K)).astype(np.uint8)
    ws = r.uniform(0.01, 0.1, size=(2, 2)).astype(np.float32)
    y, codes, xs = quant.linear_a8w8_quant(x, wq, ws)
    assert np.array_equal(y, oracle.linear_a8w8_block(codes, xs, wq, ws))
    # and within the quantisation error of the bf16 product of the dequantised weight
    wd = formats.dec_e4m3fn(wq) * ws[np.arange(N) // 128][:, np.arange(K) // 128]
    exact = formats.dec_bf16(x) @ wd.T
    assert np.linalg.norm(y - exact) / np.linalg.norm(exact) < 0.05


def _half_away(v):
    v = np.clip(np.asarray(v, dtype=np.float64), -448, 448)
    a = np.abs(v)
    m, e = np.frexp(a)
    q = np.where(a >= 2.0 ** -6, np.ldexp(np.floor(np.ldexp(m, 4) + 0.5), e - 4), np.floor(a * 512 + 0.5) / 512)
    idx = np.searchsorted(quant._POS_VALUES, q).astype(np.uint8)
    return np.where((v < 0) & (idx != 0), idx | 0x80, idx).astype(np.uint8)


def _truncating(v):
    v = np.clip(np.asarray(v, dtype=np.float64), -448, 448)
    a = np.abs(v)
    m, e = np.frexp(a)
    q = np.where(a >= 2.0 ** -6, np.ldexp(np.floor(np.ldexp(m, 4)), e - 4), np.floor(a * 512) / 512)
    idx = np.searchsorted(quant._POS_VALUES, q).astype(np.uint8)
    return np.where((v < 0) & (idx != 0), idx | 0x80, idx).astype(np.uint8)


def _no_clamp(v):
    v = np.asarray(v, dtype=np.float64)
    out = quant.e4m3fn_rne_bits(v)
    return np.where(np.abs(v) > 448, 0x7F | (out & 0x80), out).astype(np.uint8)


@pytest.mark.parametrize("mutant", [_half_away, _truncating, _no_clamp])
def test_encoder_pins_catch_mistakes(mutant):
    assert grid_pins(mutant) != []


def _q_wrong_divisor(bits):
    x = formats.dec_bf16(bits).astype(np.float32)
    M, K = x.shape
    G = -(-K // 128)
    c = np.empty((M, K), np.uint8)
    s = np.empty((M, G), np.float32)
    for g in range(G):
        b = x[:, g * 128:(g + 1) * 128]
        a = np.max(np.abs(b), axis=1)
        sg = np.where(a > 0, a / np.float32(240.0), 1).astype(np.float32)   # the e4m3fnuz maximum
        c[:, g * 128:(g + 1) * 128] = quant.e4m3fn_rne_bits((b / sg[:, None]).astype(np.float64))
        s[:, g] = sg
    return c, s


def _q_row_scale(bits):
    x = formats.dec_bf16(bits).astype(np.float32)
    a = np.max(np.abs(x), axis=1)
    sg = np.where(a > 0, a / np.float32(448.0), 1).astype(np.float32)      # one scale per row
    c = quant.e4m3fn_rne_bits((x / sg[:, None]).astype(np.float64))
    G = -(-x.shape[1] // 128)
    return c, np.repeat(sg[:, None], G, axis=1)


def _q_zero_scale(bits):
    c, s = quant.quantize_a8w8_x(bits)
    return c, np.where(s == 1.0, np.float32(0.0), s)


@pytest.mark.parametrize("mutant", [_q_wrong_divisor, _q_row_scale, _q_zero_scale])
def test_quantiser_pins_catch_mistakes(mutant):
    assert quant_pins(mutant) != []

"""Pins of the oracle's format decoders and its bf16 rounding against routes
that do not share its code: torch's CPU casts, the OCP/IEEE anchor tables under
tests/golden, and exact rational arithmetic."""
import math
import os
from fractions import Fraction

import numpy as np
import torch

from oracle import E4M3FN_TABLE, bf16_rne_bits, dec_bf16, dec_e4m3fn

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _anchors(name):
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                code, val = line.split()
                out.append((int(code, 16), float(val)))
    return out


def _same(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    both_nan = np.isnan(a) & np.isnan(b)
    eq = (a == b) & (np.signbit(a) == np.signbit(b))
    return bool(np.all(both_nan | eq))


def test_bf16_exhaustive_vs_torch():
    codes = np.arange(65536, dtype=np.uint32)
    mine = dec_bf16(codes)
    t = torch.from_numpy(codes.astype(np.uint16).view(np.int16)).view(torch.bfloat16)
    ref = t.to(torch.float64).numpy()
    assert _same(mine, ref)


def test_bf16_anchors():
    for code, val in _anchors("bf16_anchors.txt"):
        got = float(dec_bf16(np.array([code]))[0])
        if math.isnan(val):
            assert math.isnan(got), hex(code)
        else:
            assert got == val and math.copysign(1, got) == math.copysign(1, val), hex(code)


def test_e4m3fn_exhaustive_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert _same(dec_e4m3fn(codes), ref)
    assert _same(E4M3FN_TABLE, ref)


def test_e4m3fn_anchors_and_structure():
    for code, val in _anchors("e4m3fn_anchors.txt"):
        got = float(dec_e4m3fn(np.array([code]))[0])
        if math.isnan(val):
            assert math.isnan(got), hex(code)
        else:
            assert got == val and math.copysign(1, got) == math.copysign(1, val), hex(code)
    finite = E4M3FN_TABLE[np.isfinite(E4M3FN_TABLE)]
    assert finite.size == 254 and finite.max() == 448.0 and finite.min() == -448.0
    # positive codes are strictly increasing in value
    pos = E4M3FN_TABLE[:0x7F]
    assert np.all(np.diff(pos) > 0)
    # every e4m3fn value is exactly a bf16 value (7 fraction bits >= 3)
    back = dec_bf16(bf16_rne_bits(finite))
    assert np.array_equal(back, finite)


def test_bf16_rne_matches_torch_on_float32():
    r = np.random.default_rng(123)
    v = r.standard_normal(200_000).astype(np.float32) * np.float32(3.0)
    v = np.concatenate([v, (r.standard_normal(1000) * 1e-39).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, 65504.0, 3.0e38, -3.0e38], np.float32)])
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16_rne_bits(v.astype(np.float64)), ref)


def test_bf16_rne_ties_and_single_rounding():
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa (1.0) wins.
    assert dec_bf16(bf16_rne_bits(np.array([1 + 2.0 ** -8])))[0] == 1.0
    # 1 + 3*2^-8 is a tie between 1+2^-7 (odd) and 1+2^-6 (even): rounds up.
    assert dec_bf16(bf16_rne_bits(np.array([1 + 3 * 2.0 ** -8])))[0] == 1 + 2.0 ** -6
    # just above the tie rounds up; a float32 detour would round the tiny
    # excess away first and then tie down to 1.0 (double rounding).
    v = 1 + 2.0 ** -8 + 2.0 ** -40
    assert dec_bf16(bf16_rne_bits(np.array([v])))[0] == 1 + 2.0 ** -7
    # exact by rational comparison on random doubles: the result is the
    # nearest bf16 value
    r = np.random.default_rng(7)
    xs = r.standard_normal(300) * 10.0
    got = dec_bf16(bf16_rne_bits(xs))
    for x, g in zip(xs, got):
        fx, fg = Fraction(float(x)), Fraction(float(g))
        mant, ex = math.frexp(float(g)) if g != 0 else (0.5, 0)
        ulp = Fraction(2) ** (ex - 8)
        assert abs(fx - fg) <= ulp / 2
    assert np.isinf(dec_bf16(bf16_rne_bits(np.array([3.5e38])))[0])

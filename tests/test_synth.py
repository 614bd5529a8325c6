"""The seeded generators: determinism, thread-count independence, encodings and
quantisation rules, and the sizes the pages print."""
import os

import numpy as np

import oracle
import synth
from synth import gen


def _golden():
    d = {}
    with open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                k, *v = line.split()
                d.setdefault(k, []).append([float(t) for t in v])
    return d


def test_deterministic_and_chunk_layout(monkeypatch):
    a = synth.normal_f32(0, 2, (3, gen.CHUNK // 2 + 5))
    b = synth.normal_f32(0, 2, (3, gen.CHUNK // 2 + 5))
    assert np.array_equal(a, b)
    monkeypatch.setattr(gen, "_threads", lambda: 1)
    c = synth.normal_f32(0, 2, (3, gen.CHUNK // 2 + 5))
    assert np.array_equal(a, c)
    # a different tensor id or seed gives a different stream
    assert not np.array_equal(a, synth.normal_f32(0, 3, a.shape))
    assert not np.array_equal(a, synth.normal_f32(1, 2, a.shape))
    # the first chunk equals a plain float64 draw of that stream, scaled
    first = np.random.default_rng([0, 2, 0]).standard_normal(1000)
    assert np.array_equal(synth.normal_f32(0, 2, (1000,)), first.astype(np.float32))


def test_distribution_moments():
    v = synth.normal_f32(0, 2, (1 << 20,), 0.02).astype(np.float64)
    assert abs(v.mean()) < 1e-4 and abs(v.std() - 0.02) < 1e-4


def test_bf16_and_fp8_encoders_round_to_nearest():
    r = np.random.default_rng(5)
    v = r.standard_normal(10000).astype(np.float32)
    bits = synth.bf16_bits(v)
    assert np.array_equal(bits, oracle.bf16_rne_bits(v.astype(np.float64)))
    q = synth.e4m3fn_bytes(v * 100)
    d = oracle.dec_e4m3fn(q)
    assert np.isfinite(d).all() and np.abs(d).max() <= 448
    # nearest: no other finite code is closer than the chosen one
    table = oracle.E4M3FN_TABLE[np.isfinite(oracle.E4M3FN_TABLE)]
    tgt = np.clip(v[:500].astype(np.float64) * 100, -448, 448)
    best = np.min(np.abs(table[None, :] - tgt[:, None]), axis=1)
    assert np.all(np.abs(d[:500] - tgt) <= best + 1e-12)


def test_fp8_tensor_quantiser():
    p = synth.make_fp8_tensor(2, 300, 256, seed=0)
    assert p.w.dtype == np.uint8 and p.w.shape == (300, 256)
    wf = synth.normal_f32(0, 2, (300, 256), 0.02)
    assert p.s0.dtype == np.float32 and p.s0[0] == np.float32(np.abs(wf).max()) / np.float32(448)
    d = oracle.dec_e4m3fn(p.w) * np.float64(p.s0[0])
    assert np.isfinite(d).all()
    # dequantised weights approximate the drawn ones to e4m3's half-ulp (2^-4 rel)
    assert np.max(np.abs(d - wf) / (np.abs(wf) + p.s0[0] * 2 ** -9)) <= 2 ** -4 + 1e-6
    assert np.abs(oracle.dec_e4m3fn(p.w)).max() == 448.0


def test_a8w8_quantiser_layout():
    p = synth.make_a8w8_block(3, 256, 384, seed=0)
    assert p.x.shape == (3, 384) and p.s0.shape == (3, 3)
    assert p.w.shape == (256, 384) and p.s1.shape == (2, 3)
    xf = synth.normal_f32(0, 1, (3, 384))
    for m in range(3):
        for g in range(3):
            blk = xf[m, g * 128:(g + 1) * 128]
            assert p.s0[m, g] == np.float32(np.abs(blk).max()) / np.float32(448)
    wf = synth.normal_f32(0, 2, (256, 384), 0.02)
    assert p.s1[1, 2] == np.float32(np.abs(wf[128:, 256:]).max()) / np.float32(448)
    xd, wd = oracle.dequant_a8w8(p.x, p.s0, p.w, p.s1)
    assert np.max(np.abs(xd - xf)) <= np.max(p.s0) * 448 * 2 ** -4


def test_gated_layout():
    p = synth.make_gated(2, 5, 64)
    assert p.w.shape == (10, 64)
    assert np.array_equal(p.w[:5], synth.bf16_bits(synth.normal_f32(0, 2, (5, 64), 0.02)))
    assert np.array_equal(p.w[5:], synth.bf16_bits(synth.normal_f32(0, 3, (5, 64), 0.02)))


def test_page_figures():
    g = _golden()
    rows, cols = int(g["head_rows"][0][0]), int(g["head_cols"][0][0])
    assert (rows, cols) == synth.HEAD_NK
    gb = rows * cols * np.dtype(np.uint8).itemsize / 1e9
    assert g["head_fp8_bytes_gb_min"][0][0] <= gb <= g["head_fp8_bytes_gb_max"][0][0]
    assert sorted(tuple(int(v) for v in s) for s in g["a8w8_shape"]) == sorted(synth.A8W8_NK)
    assert g["e4m3fn_max"][0][0] == gen.E4M3_MAX == np.nanmax(oracle.E4M3FN_TABLE)


def test_rows_of():
    r = synth.rows_of(1000, 50)
    assert r[0] == 0 and r[-1] == 999 and np.all(np.diff(r) > 0)
    assert np.array_equal(r, synth.rows_of(1000, 50))

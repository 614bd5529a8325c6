"""The oracle against its pins, and the pins against planted mistakes."""
import numpy as np
import pytest

import oracle
from oracle import formats
from pins import pins_a8w8_block, pins_bf16, pins_fp8_tensor, pins_gated


def test_bf16_pins():
    assert pins_bf16(oracle.linear_bf16) == []


def test_gated_pins():
    assert pins_gated(oracle.linear_gated) == []


def test_fp8_tensor_pins():
    assert pins_fp8_tensor(oracle.linear_fp8_tensor) == []


def test_a8w8_pins():
    assert pins_a8w8_block(oracle.linear_a8w8_block) == []


def test_silu_closed_forms():
    g = np.array([0.0, 1.0, -1.0, 30.0, -800.0, 800.0])
    s = formats.silu(g)
    assert s[0] == 0.0
    assert abs(s[1] - 0.7310585786300049) < 1e-16
    assert abs(s[2] + 0.2689414213699951) < 1e-16
    assert np.isfinite(s).all() and s[4] == -0.0 or abs(s[4]) < 1e-300
    assert s[5] == 800.0
    t = np.linspace(-20, 20, 401)
    assert np.allclose(formats.silu(t) - formats.silu(-t), t, rtol=0, atol=1e-13)


def test_a8w8_grouped_form_equals_dequantised_product():
    """The per-group form sum_g xs*ws*(sum_{k in g} xq*wq) equals the dense
    product of the dequantised operands (within float64 rounding)."""
    r = np.random.default_rng(3)
    M, N, K = 3, 256, 384
    xq = r.integers(0, 0x7E, size=(M, K)).astype(np.uint8)
    wq = r.integers(0, 0x7E, size=(N, K)).astype(np.uint8)
    xs = r.uniform(0.5, 2, size=(M, 3)).astype(np.float32)
    ws = r.uniform(0.01, 0.1, size=(2, 3)).astype(np.float32)
    y = oracle.linear_a8w8_block(xq, xs, wq, ws)
    xd, wd = formats.dec_e4m3fn(xq), formats.dec_e4m3fn(wq)
    alt = np.zeros((M, N))
    for g in range(3):
        sl = slice(g * 128, (g + 1) * 128)
        part = xd[:, sl] @ wd[:, sl].T
        alt += xs[:, g:g + 1].astype(np.float64) * ws[np.arange(N) // 128, g][None, :].astype(np.float64) * part
    assert np.allclose(y, alt, rtol=1e-12, atol=0)


def test_parity_bar_semantics():
    ref = np.array([[1.0, -2.0, 0.5]])
    bits = oracle.bf16_rne_bits(ref)
    assert oracle.parity(bits, ref).ok
    bad = ref.copy()
    bad[0, 1] = -2.0 * (1 + 2 ** -5)
    assert not oracle.parity(oracle.bf16_rne_bits(bad), ref).ok
    nan = bits.copy()
    nan[0, 0] = 0x7FC0
    assert not oracle.parity(nan, ref).ok
    z = np.zeros((2, 2))
    assert oracle.parity(oracle.bf16_rne_bits(z), z).ok
    assert not oracle.parity(oracle.bf16_rne_bits(z + 1e-3), z).ok
    assert oracle.parity(np.zeros((0, 4), np.uint16), np.zeros((0, 4))).ok


# ------------------------------------------------- planted mistakes must fail
def _mut_bf16_transposed(x, w, cols=None):
    return formats.dec_bf16(x) @ formats.dec_bf16(w)          # W used as [K, N]


def _mut_bf16_dropped_term(x, w, cols=None):
    return formats.dec_bf16(x)[:, :-1] @ formats.dec_bf16(w)[:, :-1].T


def _mut_bf16_sign(x, w, cols=None):
    xd = formats.dec_bf16(x).copy()
    xd[:, 0] = -xd[:, 0]
    y = xd @ formats.dec_bf16(w).T
    return y if cols is None else y[:, cols]


def _mut_gated_swapped(x, w, cols=None):
    N = w.shape[0] // 2
    xd, wd = formats.dec_bf16(x), formats.dec_bf16(w)
    return formats.silu(xd @ wd[N:].T) * (xd @ wd[:N].T)


def _mut_gated_sigmoid(x, w, cols=None):
    N = w.shape[0] // 2
    xd, wd = formats.dec_bf16(x), formats.dec_bf16(w)
    g = xd @ wd[:N].T
    return 1 / (1 + np.exp(-g)) * (xd @ wd[N:].T)


def _mut_gated_interleaved(x, w, cols=None):
    xd, wd = formats.dec_bf16(x), formats.dec_bf16(w)
    return formats.silu(xd @ wd[0::2].T) * (xd @ wd[1::2].T)


def _mut_fp8_noscale(x, wq, s, cols=None):
    return formats.dec_bf16(x) @ formats.dec_e4m3fn(wq).T


def _mut_fp8_divscale(x, wq, s, cols=None):
    return (formats.dec_bf16(x) @ formats.dec_e4m3fn(wq).T) / float(s[0])


def _fnuz(code):
    code = np.asarray(code).astype(np.int64)
    s = np.where(code & 0x80, -1.0, 1.0)
    e = (code >> 3) & 0xF
    m = code & 7
    v = np.where(e == 0, m * 2.0 ** -10, (1 + m / 8) * 2.0 ** (e - 8))
    return s * v


def _mut_fp8_fnuz(x, wq, s, cols=None):
    return float(s[0]) * (formats.dec_bf16(x) @ _fnuz(wq).T)


def _mut_a8w8_ws_transposed(xq, xs, wq, ws, cols=None):
    K = xq.shape[1]
    N = wq.shape[0]
    kg = np.arange(K) // 128
    xd = formats.dec_e4m3fn(xq) * xs[:, kg]
    wst = ws.T
    ni = np.minimum(np.arange(N) // 128, wst.shape[0] - 1)
    kj = np.minimum(kg, wst.shape[1] - 1)
    wd = formats.dec_e4m3fn(wq) * wst[ni[:, None], kj[None, :]]
    y = xd @ wd.T
    return y if cols is None else y[:, cols]


def _mut_a8w8_block64(xq, xs, wq, ws, cols=None):
    K, N = xq.shape[1], wq.shape[0]
    kg = np.minimum(np.arange(K) // 64, xs.shape[1] - 1)
    xd = formats.dec_e4m3fn(xq) * xs[:, kg]
    ni = np.minimum(np.arange(N) // 64, ws.shape[0] - 1)
    wd = formats.dec_e4m3fn(wq) * ws[ni[:, None], np.minimum(np.arange(K) // 64, ws.shape[1] - 1)[None, :]]
    y = xd @ wd.T
    return y if cols is None else y[:, cols]


def _mut_a8w8_no_xs(xq, xs, wq, ws, cols=None):
    return oracle.linear_a8w8_block(xq, np.ones_like(xs), wq, ws, cols=cols)


@pytest.mark.parametrize("pins,mutant", [
    (pins_bf16, _mut_bf16_transposed),
    (pins_bf16, _mut_bf16_dropped_term),
    (pins_bf16, _mut_bf16_sign),
    (pins_gated, _mut_gated_swapped),
    (pins_gated, _mut_gated_sigmoid),
    (pins_gated, _mut_gated_interleaved),
    (pins_fp8_tensor, _mut_fp8_noscale),
    (pins_fp8_tensor, _mut_fp8_divscale),
    (pins_fp8_tensor, _mut_fp8_fnuz),
    (pins_a8w8_block, _mut_a8w8_ws_transposed),
    (pins_a8w8_block, _mut_a8w8_block64),
    (pins_a8w8_block, _mut_a8w8_no_xs),
])
def test_planted_mistakes_fail_a_pin(pins, mutant):
    try:
        fails = pins(mutant)
    except Exception as e:                      # a crash also counts as caught
        fails = [repr(e)]
    assert fails, f"{mutant.__name__} passed every pin"

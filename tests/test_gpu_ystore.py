"""Output stores.  The kernels write four outputs of a row with one 8-byte store
when N is a multiple of 4 and y is 8-byte aligned, and one 2-byte store each
otherwise.  y itself needs only bf16 alignment, so a y two bytes past an
aligned address must get the same bits as an aligned one, from every variant
and from table dispatch of every form, and no byte around it may change."""
import numpy as np
import pytest
import torch

import gemv_skinny_gemm_02_amd as skg
import synth
from gpu_util import ensure_workspace, host_bits, run, run_packed, say, to_device, to_device_packed

pytestmark = pytest.mark.gpu

N, K = 512, 1024
GUARD = 0x7FC1          # a bf16 NaN pattern no call writes


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    skg.load()
    ensure_workspace()


def _unaligned(M):
    """(y view of shape (M, N) at 2 bytes past a 256-byte aligned base, buffer)."""
    buf = torch.full((M * N + 8,), GUARD, dtype=torch.int16, device="cuda")
    y = buf[1:1 + M * N].view(torch.bfloat16).view(M, N)
    assert y.data_ptr() % 8 == 2
    return y, buf


def _check(tag, y_al, y_off, buf, M):
    torch.cuda.synchronize()
    a, b = host_bits(y_al), host_bits(y_off)
    assert np.array_equal(a, b), f"{tag}: unaligned y differs in {(a != b).sum()} outputs"
    g = buf.cpu().numpy().view(np.uint16)
    assert g[0] == GUARD and (g[1 + M * N:] == GUARD).all(), f"{tag}: a store left y"


@pytest.mark.parametrize("kind", ["bf16", "a8w8_block"])
@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("M", [1, 40, 256])
def test_every_variant_unaligned_y(kind, packed, M):
    p = getattr(synth, "make_" + kind)(M, N, K, seed=5)
    op = kind + ("_packed" if packed else "")
    dev = to_device_packed(p) if packed else to_device(p)
    go = run_packed if packed else run
    n = 0
    for i, name in enumerate(skg.variants(op)):
        if not skg.skinny_gemm_variant_supports(op, i, M):
            continue
        say(f"case {op} M={M} {name}")
        y_al = go(p, dev, variant=name)
        y_off, buf = _unaligned(M)
        go(p, dev, variant=name, y=y_off)
        _check(f"{op} M={M} {name}", y_al, y_off, buf, M)
        n += 1
    assert n > 0


@pytest.mark.parametrize("kind", ["bf16", "gated", "fp8_tensor", "a8w8_block", "a8w8_quant"])
@pytest.mark.parametrize("M", [1, 16, 128])
def test_dispatch_unaligned_y(kind, M):
    p = getattr(synth, "make_" + kind)(M, N, K, seed=6)
    for packed in (False, True):
        dev = to_device_packed(p) if packed else to_device(p)
        go = run_packed if packed else run
        y_al = go(p, dev)
        y_off, buf = _unaligned(M)
        go(p, dev, y=y_off)
        _check(f"{kind}{'_packed' if packed else ''} M={M}", y_al, y_off, buf, M)

"""Seeded generators.  See the package docstring for the recipe."""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np
import torch

CHUNK = 1 << 22          # elements per independent random stream
BLOCK = 128              # fp8 scale block edge (x: 1 x BLOCK, W: BLOCK x BLOCK)
E4M3_MAX = 448.0         # largest finite OCP e4m3fn value

TID_X, TID_W, TID_WU = 1, 2, 3

# Shape sets of the workloads (rows M of the decode linear, W as [N, K]).
CONFIG1 = (1, 4096, 4096)
SWEEP_M = (1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 64, 96, 128)
# mid-M rows (speculative verification and drafting) on the same (N, K)
MID_M = (144, 192, 256, 384, 512)
# small-N bf16 weights (too few rows to fill the CUs by N-split alone)
SMALLN_NK = ((64, 4096), (256, 4096), (512, 4096), (1024, 4096), (2048, 4096))
SMALLN_M = (1, 4, 8, 16, 32, 64, 128)
SWEEP_NK = ((4096, 4096), (6144, 4096), (4096, 12288), (2048, 2048), (1024, 1024))
GATED_M = (1, 3, 6, 8, 12, 16, 32)
GATED_NK = (12288, 4096)            # per half: Wg and Wu are each [N, K]
HEAD_M = (1, 2, 3, 4)
HEAD_NK = (248320, 4096)
A8W8_M = (1, 2, 4, 8, 16, 32, 64)
A8W8_NK = ((32768, 1024), (8192, 4096))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_f32(seed: int, tid: int, shape, std: float = 1.0) -> np.ndarray:
    """float32 array of N(0, std^2) draws for tensor ``tid`` (row-major)."""
    shape = tuple(int(s) for s in shape)
    total = int(np.prod(shape)) if shape else 1
    out = np.empty(total, dtype=np.float32)
    nchunks = (total + CHUNK - 1) // CHUNK

    def fill(c: int) -> None:
        lo = c * CHUNK
        hi = min(total, lo + CHUNK)
        r = np.random.default_rng([seed, tid, c])
        v = r.standard_normal(hi - lo)
        if std != 1.0:
            v *= std
        out[lo:hi] = v

    if nchunks <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) of float32 values, round-to-nearest-even."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def e4m3fn_bytes(a: np.ndarray) -> np.ndarray:
    """OCP e4m3fn bytes (uint8) of float32 values, clamped to +-448 then RNE."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    t = t.clamp(-E4M3_MAX, E4M3_MAX)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _amax_scale(amax: np.ndarray) -> np.ndarray:
    amax = amax.astype(np.float32)
    s = amax / np.float32(E4M3_MAX)
    return np.where(amax > 0, s, np.float32(1.0)).astype(np.float32)


@dataclass
class Problem:
    """One call's inputs.  ``x``/``w`` are raw bits; scales are float32."""
    kind: str
    M: int
    N: int
    K: int
    x: np.ndarray
    w: np.ndarray
    s0: np.ndarray | None = None       # fp8 tensor: w_scale[1]; a8w8: xs[M, K/128]
    s1: np.ndarray | None = None       # a8w8 (both forms): ws[N/128, K/128]
    meta: dict = field(default_factory=dict)


def make_bf16(M: int, N: int, K: int, seed: int = 0) -> Problem:
    x = bf16_bits(normal_f32(seed, TID_X, (M, K), 1.0))
    w = bf16_bits(normal_f32(seed, TID_W, (N, K), 0.02))
    return Problem("bf16", M, N, K, x, w)


def make_gated(M: int, N: int, K: int, seed: int = 0) -> Problem:
    """W is one [2N, K] buffer: rows [0, N) are the gate, [N, 2N) the up half."""
    x = bf16_bits(normal_f32(seed, TID_X, (M, K), 1.0))
    wg = bf16_bits(normal_f32(seed, TID_W, (N, K), 0.02))
    wu = bf16_bits(normal_f32(seed, TID_WU, (N, K), 0.02))
    return Problem("gated", M, N, K, x, np.concatenate([wg, wu], axis=0))


def make_fp8_tensor(M: int, N: int, K: int, seed: int = 0) -> Problem:
    x = bf16_bits(normal_f32(seed, TID_X, (M, K), 1.0))
    wf = normal_f32(seed, TID_W, (N, K), 0.02)
    amax = np.float32(np.abs(wf).max()) if wf.size else np.float32(0)
    s = _amax_scale(np.array([amax]))
    wq = np.empty((N, K), dtype=np.uint8)
    step = 8192
    for lo in range(0, N, step):                 # bounded temporaries
        wq[lo:lo + step] = e4m3fn_bytes(wf[lo:lo + step] / s[0])
    del wf
    return Problem("fp8_tensor", M, N, K, x, wq, s0=s)


def _block_quant(a: np.ndarray, rb: int, cb: int):
    """Quantise a [R, C] float32 array with one scale per rb x cb block."""
    R, C = a.shape
    nrb, ncb = -(-R // rb), -(-C // cb)
    scales = np.empty((nrb, ncb), dtype=np.float32)
    q = np.empty((R, C), dtype=np.uint8)
    for i in range(nrb):
        r0, r1 = i * rb, min(R, (i + 1) * rb)
        for j in range(ncb):
            c0, c1 = j * cb, min(C, (j + 1) * cb)
            blk = a[r0:r1, c0:c1]
            sc = _amax_scale(np.array([np.abs(blk).max() if blk.size else 0.0]))[0]
            scales[i, j] = sc
            q[r0:r1, c0:c1] = e4m3fn_bytes(blk / sc)
    return q, scales


def _group_quant_rows(a: np.ndarray, g: int):
    """Quantise a [R, C] float32 array with one scale per row per g columns."""
    R, C = a.shape
    ng = -(-C // g)
    scales = np.empty((R, ng), dtype=np.float32)
    q = np.empty((R, C), dtype=np.uint8)
    for j in range(ng):
        c0, c1 = j * g, min(C, (j + 1) * g)
        blk = a[:, c0:c1]
        amax = np.abs(blk).max(axis=1) if blk.size else np.zeros(R, np.float32)
        sc = _amax_scale(amax)
        scales[:, j] = sc
        q[:, c0:c1] = e4m3fn_bytes(blk / sc[:, None])
    return q, scales


def make_a8w8_block(M: int, N: int, K: int, seed: int = 0) -> Problem:
    xf = normal_f32(seed, TID_X, (M, K), 1.0)
    wf = normal_f32(seed, TID_W, (N, K), 0.02)
    xq, xs = _group_quant_rows(xf, BLOCK)
    wq, ws = _block_quant(wf, BLOCK, BLOCK)
    return Problem("a8w8_block", M, N, K, xq, wq, s0=xs, s1=ws)


def make_a8w8_quant(M: int, N: int, K: int, seed: int = 0) -> Problem:
    """A8W8 block scale with bf16 x (the call quantises it): x as make_bf16's,
    W and its 128x128 block scales as make_a8w8_block's."""
    x = bf16_bits(normal_f32(seed, TID_X, (M, K), 1.0))
    wf = normal_f32(seed, TID_W, (N, K), 0.02)
    wq, ws = _block_quant(wf, BLOCK, BLOCK)
    return Problem("a8w8_quant", M, N, K, x, wq, s0=None, s1=ws)


def rows_of(n_total: int, count: int, seed: int = 0) -> np.ndarray:
    """A seeded, sorted sample of output columns (rows of W) to spot-check,
    always including the first and last row."""
    count = min(count, n_total)
    r = np.random.default_rng([seed, 99])
    pick = r.choice(n_total, size=count, replace=False)
    pick[0], pick[-1] = 0, n_total - 1
    return np.unique(pick).astype(np.int64)

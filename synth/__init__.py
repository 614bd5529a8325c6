"""Seeded synthetic inputs for the skinny decode linear, shared by the oracle's
tests and the GPU path's tests and benchmark.

This module only draws random numbers and encodes them into the storage
formats the linear consumes (bf16 bits, OCP e4m3fn bytes, fp32 scales).  It
holds none of the linear's arithmetic: no products, no sums, no activation.

Recipe (the workloads of the decode-linear pages: Qwen3.5 decode linears and
its 248k x 4096 vocabulary head, DeepSeek-V4-flash's A8W8 block-scale layers):

* every tensor has its own stream.  A tensor of E elements is cut into chunks
  of ``CHUNK`` elements in row-major order; chunk c of tensor ``tid`` is drawn
  from ``numpy.random.default_rng([seed, tid, c]).standard_normal`` in float64
  and scaled by the tensor's standard deviation, then rounded once to float32.
  Chunking makes generation parallel and independent of the thread count.
* tensor ids: x = 1, W (or the gate half Wg) = 2, the up half Wu = 3.
* x ~ N(0, 1), W ~ N(0, 0.02) (0.02 is a standard deviation).
* bf16 tensors: float32 -> bf16 round-to-nearest-even (torch's CPU cast).
* fp8 tensors (OCP e4m3fn, largest finite 448): a scale is amax/448 over the
  scale's block (whole tensor; 1 x 128 groups of a row of x; 128 x 128 blocks
  of W), computed in float32, 1.0 when the block is all zero; the stored byte is
  RNE(clamp(v / scale, -448, 448)) via torch's CPU float8_e4m3fn cast.
* the A8W8 form with x quantised inside the call takes x as bf16 (as above)
  and W with its block scales as the A8W8 form does.
"""
from .gen import (CHUNK, normal_f32, bf16_bits, e4m3fn_bytes, make_bf16,
                  make_gated, make_fp8_tensor, make_a8w8_block, make_a8w8_quant, BLOCK,
                  rows_of, SWEEP_M, MID_M, SMALLN_NK, SMALLN_M, SWEEP_NK, GATED_M, GATED_NK, HEAD_M,
                  HEAD_NK, A8W8_M, A8W8_NK, CONFIG1)

__all__ = ["CHUNK", "normal_f32", "bf16_bits", "e4m3fn_bytes", "make_bf16",
           "make_gated", "make_fp8_tensor", "make_a8w8_block", "make_a8w8_quant", "BLOCK",
           "rows_of", "SWEEP_M", "MID_M", "SMALLN_NK", "SMALLN_M", "SWEEP_NK", "GATED_M", "GATED_NK", "HEAD_M",
           "HEAD_NK", "A8W8_M", "A8W8_NK", "CONFIG1"]

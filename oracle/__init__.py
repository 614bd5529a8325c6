"""CPU oracle for the decode-shaped skinny linear  y[M,N] = x[M,K] . W[N,K]^T.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this package: only the test suite, the smoke check of the package entry file
and the benchmark's CPU-baseline leg do.  It shares no code, table or helper
with the HIP library; the only thing both sides use is the seeded input
generator package ``synth``, which holds none of the linear's arithmetic.

What it computes is the plain definition of each of the four forms, in float64
over the exact values that the stored bits encode.  The forms, as the pages name
them:

* bf16 decode linear ("decode linears", "skinny GEMM", "GEMV" -- mstar PR #1104,
  section "Why");
* fused gate/up, silu(x Wg^T) * (x Wu^T) ("decode_gemv_silu_mul", "A fused
  gate/up has its own gated1- entry" -- mstar PR #1104, "Why" and "What
  changed");
* an fp8 weight with one scale for the whole tensor (the fp8 draft head --
  mstar PR #1102, "What changed", draft_head: fp8 bullet);
* A8W8 with block scales (Decode optimization round 3, "Retained change
  2: decode-M rows for the A8W8 bpreshuffle table"), and the same with the
  activation quantisation folded in (``quant.py``; the same page leaves that
  fusion as open work in "Rejected paths").

Every function below is pinned by the CPU tests against brute force in exact
rational arithmetic, exhaustive format tables checked against torch's casts,
closed forms and exact invariants.
"""
from .formats import (dec_bf16, dec_e4m3fn, E4M3FN_TABLE, bf16_rne_bits,
                      silu)
from .linear import (linear_bf16, linear_gated, linear_fp8_tensor,
                     linear_a8w8_block, dequant_a8w8, BLOCK)
from .check import parity, ParityResult, TOL_MAX_REL, TOL_FRO
from .quant import e4m3fn_rne_bits, quantize_a8w8_x, linear_a8w8_quant, E4M3_MAX

__all__ = ["dec_bf16", "dec_e4m3fn", "E4M3FN_TABLE", "bf16_rne_bits", "silu",
           "linear_bf16", "linear_gated", "linear_fp8_tensor",
           "linear_a8w8_block", "dequant_a8w8", "BLOCK", "parity",
           "ParityResult", "TOL_MAX_REL", "TOL_FRO", "e4m3fn_rne_bits",
           "quantize_a8w8_x", "linear_a8w8_quant", "E4M3_MAX"]

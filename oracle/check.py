"""Parity bar between a bf16 result and the float64 oracle.  Test
infrastructure only.

The bar: max |y - y_ref| <= 2^-7 * max |y_ref|, relative Frobenius error
||y - y_ref|| / ||y_ref|| <= 5e-3, no NaN or Inf; when y_ref is all zero, y must
be exactly zero.  Several summation orders are equally correct (the pages
record different vendor reduction orders differing at a relative L2 of up to
6e-5 -- Decode optimization round 3, "Rejected paths", TunableOp bullet),
so the bar is a tolerance, not bit equality.  Rounding the exact result once to
bf16 already costs up to 2^-9 relative per element, a quarter of the max-abs
budget.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .formats import dec_bf16

TOL_MAX_REL = 2.0 ** -7
TOL_FRO = 5e-3


@dataclass
class ParityResult:
    ok: bool
    max_abs_err: float
    max_ref: float
    rel_fro: float
    nonfinite: int
    msg: str

    def __bool__(self) -> bool:
        return self.ok


def parity(y_bits, y_ref, tol_max_rel: float = TOL_MAX_REL,
           tol_fro: float = TOL_FRO) -> ParityResult:
    """Compare bf16 bits ``y_bits`` with float64 ``y_ref`` (same shape)."""
    y = dec_bf16(y_bits)
    ref = np.asarray(y_ref, dtype=np.float64)
    if y.shape != ref.shape:
        return ParityResult(False, np.inf, np.nan, np.inf, 0,
                            f"shape {y.shape} != {ref.shape}")
    nonfinite = int(np.count_nonzero(~np.isfinite(y)))
    if y.size == 0:
        return ParityResult(True, 0.0, 0.0, 0.0, 0, "empty")
    max_ref = float(np.max(np.abs(ref)))
    err = np.abs(y - ref)
    max_err = float(np.max(err)) if nonfinite == 0 else np.inf
    nref = float(np.linalg.norm(ref))
    rel_fro = float(np.linalg.norm(y - ref) / nref) if nref > 0 else (0.0 if max_err == 0 else np.inf)
    if nonfinite:
        ok = False
    elif max_ref == 0.0:
        ok = max_err == 0.0
    else:
        ok = max_err <= tol_max_rel * max_ref and rel_fro <= tol_fro
    msg = (f"max|err|={max_err:.3e} (bar {tol_max_rel * max_ref:.3e}), "
           f"relF={rel_fro:.3e} (bar {tol_fro:.1e}), nonfinite={nonfinite}")
    return ParityResult(ok, max_err, max_ref, rel_fro, nonfinite, msg)

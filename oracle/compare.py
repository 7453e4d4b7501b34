"""Acceptance rules for GPU results against the float64 oracle.

Test infrastructure only.  The pages give no tolerance; the rules follow the
stated target for this GEMM:
  * integer-valued inputs (|partial sums| < 2^24, so fp32 accumulation is
    exact in any order): fp32 output must equal float32(D_ref) exactly, fp16
    output must equal rne16(D_ref) exactly; values are compared, so +0 == -0;
  * random floats, fp32 output: max |D - D_ref| <= 1e-4 * sqrt(K);
  * random floats, fp16 output: |D - D_ref| <= ulp16(D_ref) + 1e-4 * sqrt(K)
    for every element;
  * no NaN or Inf anywhere.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

from . import fp16


@dataclass
class Verdict:
    ok: bool
    rule: str
    n: int
    worst: float
    limit: float
    where: tuple

    def __str__(self):
        return (f"{'PASS' if self.ok else 'FAIL'} {self.rule}: n={self.n} "
                f"worst={self.worst:.3e} limit={self.limit:.3e} at {self.where}")


def _nonfinite(d: np.ndarray):
    bad = ~np.isfinite(d)
    if bad.any():
        idx = np.argwhere(bad)[0]
        return tuple(int(i) for i in idx)
    return None


def check(d_gpu: np.ndarray, d_ref: np.ndarray, out_dtype: str, K: int,
          integer_inputs: bool) -> Verdict:
    """Compare element by element; shapes must match."""
    d = np.asarray(d_gpu, dtype=np.float64)
    r = np.asarray(d_ref, dtype=np.float64)
    assert d.shape == r.shape, (d.shape, r.shape)
    n = d.size
    if n == 0:
        return Verdict(True, "empty", 0, 0.0, 0.0, ())
    nf = _nonfinite(d)
    if nf is not None:
        return Verdict(False, "non-finite output", n, math.inf, 0.0, nf)
    if integer_inputs:
        if out_dtype == "f32":
            want = r.astype(np.float32).astype(np.float64)
            rule = "exact float32(D_ref)"
        else:
            want = fp16.rne16_array(r)
            rule = "exact rne16(D_ref)"
        diff = np.abs(d - want)
        worst = float(diff.max())
        where = tuple(int(i) for i in np.unravel_index(int(diff.argmax()), d.shape))
        return Verdict(worst == 0.0, rule, n, worst, 0.0, where)
    tol = 1e-4 * math.sqrt(K)
    diff = np.abs(d - r)
    if out_dtype == "f32":
        worst = float(diff.max())
        where = tuple(int(i) for i in np.unravel_index(int(diff.argmax()), d.shape))
        return Verdict(worst <= tol, "max|D-Dref| <= 1e-4*sqrt(K)", n, worst, tol, where)
    lim = fp16.ulp16_array(r) + tol
    excess = diff - lim
    i = int(excess.argmax())
    where = tuple(int(x) for x in np.unravel_index(i, d.shape))
    return Verdict(bool((excess <= 0).all()), "|D-Dref| <= ulp16(Dref) + 1e-4*sqrt(K)",
                   n, float(diff.reshape(-1)[i]), float(lim.reshape(-1)[i]), where)
